"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names the kind of pin: a hand-worked example (tests/golden), a
closed-form identity, a special case that reduces to a library routine,
brute force over all subsets, or a published format definition.  Each is
chosen so that a plausible slip in the oracle (a dropped ReLU, a wrong sign,
a transposed operand, a wrong tie rule, an off-by-one in the causal range)
makes at least one of them fail.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _num(x):
    if isinstance(x, str):
        return {"ln3": math.log(3.0), "ln2": math.log(2.0), "2ln2": 2 * math.log(2.0)}[x]
    return float(x)


# ---------------------------------------------------------------- formats --

def test_e4m3_decode_matches_torch_and_spec():
    """Published format definition (OCP E4M3FN) and an independent library decoder."""
    codes = np.arange(256, dtype=np.uint8)
    mine = O.decode_e4m3(codes)
    lib = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(mine) & np.isnan(lib)
    assert np.all(both_nan | (mine == lib))
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF]) and np.isnan(mine).sum() == 2
    assert mine[0x7E] == 448.0 and mine[0xFE] == -448.0        # largest finite
    assert mine[0x01] == 2.0 ** -9                               # smallest subnormal
    assert mine[0x08] == 2.0 ** -6                               # smallest normal
    assert mine[0x38] == 1.0 and mine[0x40] == 2.0 and mine[0x44] == 3.0
    assert mine[0x80] == 0.0 and math.copysign(1.0, mine[0x80]) == -1.0


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]                       # drop inf/nan patterns
    lib = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.decode_bf16(bits), lib)


# ---------------------------------------------------------------- indexer --

def test_indexer_hand_worked_example():
    """Hand-worked example (tests/golden/worked_examples.json)."""
    g = _golden()["indexer"]
    q_I = np.array(g["q_I"], dtype=np.float64)
    w = np.array(g["w"], dtype=np.float64)
    k_I = np.array(g["k_I"], dtype=np.float64)
    rows = O.indexer_scores(q_I, w, k_I)
    assert [list(r) for r in rows] == g["scores"]
    assert O.indexer_topk(q_I, w, k_I, 2).tolist() == g["topk_k2"]
    assert O.indexer_topk(q_I, w, k_I, 1).tolist() == g["topk_k1"]


def _rand_int(rng, shape, lo=-3, hi=3):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float64)


def test_indexer_relu_identities():
    """Closed forms: relu(x) - relu(-x) = x and relu(x) + relu(-x) = |x|.

    Two heads carrying q and -q: with w = (1, -1) the score is the plain dot
    product q.k; with w = (1, 1) it is |q.k|.  Checked against a full masked
    matrix product over all (t, s).
    """
    rng = np.random.default_rng(1)
    L, d = 37, 8
    q = _rand_int(rng, (L, d))
    k_I = _rand_int(rng, (L, d))
    q_I = np.stack([q, -q], axis=1)                              # [L, 2, d]
    dense = q @ k_I.T
    for w_row, expect in (((1.0, -1.0), dense), ((1.0, 1.0), np.abs(dense))):
        w = np.tile(np.array(w_row), (L, 1))
        rows = O.indexer_scores(q_I, w, k_I)
        for t in range(L):
            assert len(rows[t]) == t + 1                         # causal, self included
            assert np.array_equal(rows[t], expect[t, : t + 1])


def test_indexer_single_head_is_gemm():
    """H_I = 1, w = 1, non-negative inputs: the score is the masked GEMM Q K^T (library matmul)."""
    rng = np.random.default_rng(2)
    L, d = 29, 16
    q = rng.random((L, d))
    k_I = rng.random((L, d))
    rows = O.indexer_scores(q[:, None, :], np.ones((L, 1)), k_I)
    ref = torch.from_numpy(q) @ torch.from_numpy(k_I).T
    for t in range(L):
        np.testing.assert_allclose(rows[t], ref[t, : t + 1].numpy(), rtol=1e-14, atol=0)


def test_indexer_weights_linear_and_zero():
    """Invariants: w = 0 gives 0; scores are linear in w (exact on integer data)."""
    rng = np.random.default_rng(3)
    L, H, d = 23, 4, 8
    q_I = _rand_int(rng, (L, H, d))
    k_I = _rand_int(rng, (L, d))
    w1 = _rand_int(rng, (L, H), 0, 3)
    w2 = _rand_int(rng, (L, H), -2, 2)
    r1 = O.indexer_scores(q_I, w1, k_I)
    r2 = O.indexer_scores(q_I, w2, k_I)
    r12 = O.indexer_scores(q_I, w1 + w2, k_I)
    r0 = O.indexer_scores(q_I, np.zeros((L, H)), k_I)
    for t in range(L):
        assert np.array_equal(r12[t], r1[t] + r2[t])
        assert not np.any(r0[t])


def test_indexer_query_offset_matches_full_prefill():
    """Chunk invariance: queries at pos0.. score the same rows as in a full prefill."""
    rng = np.random.default_rng(4)
    L, H, d, pos0 = 40, 3, 8, 25
    q_I = _rand_int(rng, (L, H, d))
    w = _rand_int(rng, (L, H), 0, 3)
    k_I = _rand_int(rng, (L, d))
    full = O.indexer_scores(q_I, w, k_I)
    tail = O.indexer_scores(q_I[pos0:], w[pos0:], k_I, pos0=pos0)
    for t in range(L - pos0):
        assert np.array_equal(tail[t], full[pos0 + t])


# ------------------------------------------------------------------ top-k --

def _brute_topk(scores, k):
    """Enumerate every k-subset; keep the largest score sum, then the lexicographically smallest set."""
    n = len(scores)
    if k >= n:
        return list(range(n))
    best = None
    for sub in itertools.combinations(range(n), k):       # generated in lexicographic order
        s = sum(scores[i] for i in sub)
        if best is None or s > best[0]:
            best = (s, list(sub))
    return best[1]


def test_topk_matches_subset_brute_force():
    """Brute force over all subsets on small integer rows with many ties."""
    rng = np.random.default_rng(5)
    for _ in range(300):
        n = int(rng.integers(1, 10))
        k = int(rng.integers(1, 6))
        row = rng.integers(-2, 3, size=n).astype(np.int64)
        got = O.topk_row(row.astype(np.float32), k)
        want = _brute_topk(row.tolist(), k)
        assert got[: len(want)].tolist() == want
        assert np.all(got[len(want):] == -1)


def test_topk_special_cases():
    n = 50
    inc = np.arange(n, dtype=np.float32)
    assert O.topk_row(inc, 7).tolist() == list(range(n - 7, n))          # increasing -> last k
    assert O.topk_row(np.zeros(n, np.float32), 7).tolist() == list(range(7))  # all equal -> first k
    assert O.topk_row(inc, 64).tolist() == list(range(n)) + [-1] * 14    # k >= n -> everything
    z = np.array([-0.0, 0.0, -0.0, 0.0], dtype=np.float32)
    assert O.topk_row(z, 2).tolist() == [0, 1]                           # -0 ties +0
    neg = np.array([-5, -1, -3, -1], dtype=np.float32)
    assert O.topk_row(neg, 2).tolist() == [1, 3]


def test_topk_decision_in_float32():
    """Two fp64 scores that round to the same float32 tie, and the lower index wins."""
    a = 1.0
    b = 1.0 + 2.0 ** -30                                           # same float32 as a
    row = O.to_decision_precision(np.array([a, b]))
    assert O.topk_row(row, 1).tolist() == [0]


# -------------------------------------------------------------- attention --

def test_attention_hand_worked_example():
    g = _golden()["attention"]
    K = np.array(g["K"], dtype=np.float64)
    V = np.array(g["V"], dtype=np.float64)
    kv = np.stack([K, V], axis=1)                                  # [3, 2, 4]
    for case in g["cases"]:
        q = np.array([[_num(x) for x in case["q"]]])               # one head
        idx = np.array(case["idx"], dtype=np.int32)
        out = O.sparse_attn_row(q, kv, idx, scale=0.5)
        np.testing.assert_allclose(out[0], case["out"], rtol=1e-13, atol=1e-13)


def test_attention_full_selection_is_dense_causal_sdpa():
    """k >= L: the sparse attention is dense causal attention (torch SDPA in fp64)."""
    rng = np.random.default_rng(6)
    L, H, d = 33, 3, 16
    q = rng.standard_normal((L, H, d))
    kv = rng.standard_normal((L, 2, d))
    idx = np.stack([O.topk_row(np.zeros(t + 1, np.float32), 64) for t in range(L)])
    out = O.sparse_attn(q, kv, idx)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]                # [1, H, L, d]
    tk = torch.from_numpy(kv[:, 0]).expand(H, L, d)[None]
    tv = torch.from_numpy(kv[:, 1]).expand(H, L, d)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    np.testing.assert_allclose(out, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_attention_closed_forms():
    rng = np.random.default_rng(7)
    Lk, H, d = 20, 4, 8
    kv = rng.standard_normal((Lk, 2, d))
    idx = np.array([3, 5, 11, 19, -1, -1], dtype=np.int32)
    # q = 0: uniform weights -> mean of the selected V rows
    out0 = O.sparse_attn_row(np.zeros((H, d)), kv, idx, 0.3)
    np.testing.assert_allclose(out0, np.tile(kv[[3, 5, 11, 19], 1].mean(0), (H, 1)), rtol=1e-13)
    # two rows: out = V_b + (V_a - V_b) * sigmoid(l_a - l_b)
    q = rng.standard_normal((H, d))
    two = np.array([2, 7, -1], dtype=np.int32)
    out2 = O.sparse_attn_row(q, kv, two, 0.25)
    la = 0.25 * q @ kv[2, 0]
    lb = 0.25 * q @ kv[7, 0]
    sig = 1.0 / (1.0 + np.exp(lb - la))
    np.testing.assert_allclose(out2, kv[7, 1] + (kv[2, 1] - kv[7, 1]) * sig[:, None], rtol=1e-12)
    # convexity: every channel lies between the selected rows' min and max
    out = O.sparse_attn_row(q, kv, idx, 1.0)
    sel = kv[[3, 5, 11, 19], 1]
    assert np.all(out >= sel.min(0) - 1e-12) and np.all(out <= sel.max(0) + 1e-12)
    # adding one vector c to every K row shifts each head's logits by a constant: no change
    kv_shift = kv.copy()
    kv_shift[:, 0] += rng.standard_normal(d)
    np.testing.assert_allclose(O.sparse_attn_row(q, kv_shift, idx, 1.0), out, rtol=1e-11)


# ------------------------------------------------------------------ stack --

def _layer(rng, L, H_I, d_I, H, d, full):
    lay = {"q": rng.standard_normal((L, H, d)), "kv": rng.standard_normal((L, 2, d))}
    if full:
        lay.update(q_I=_rand_int(rng, (L, H_I, d_I)), w=_rand_int(rng, (L, H_I), 0, 3),
                   k_I=_rand_int(rng, (L, d_I)))
    return lay


def test_stack_pattern_semantics():
    """[Skill, Step 3]: F computes and caches, S reuses the nearest preceding F, S-first is an error."""
    rng = np.random.default_rng(8)
    L, H_I, d_I, H, d, k = 48, 4, 8, 2, 8, 6
    pattern = "FSSFSS"
    layers = [_layer(rng, L, H_I, d_I, H, d, c == "F") for c in pattern]
    outs, used, calls = O.run_stack(pattern, layers, k)
    assert calls == pattern.count("F")
    f0 = O.indexer_topk(layers[0]["q_I"], layers[0]["w"], layers[0]["k_I"], k)
    f3 = O.indexer_topk(layers[3]["q_I"], layers[3]["w"], layers[3]["k_I"], k)
    for l, ref in ((0, f0), (1, f0), (2, f0), (3, f3), (4, f3), (5, f3)):
        assert np.array_equal(used[l], ref)
        assert np.array_equal(outs[l], O.sparse_attn(layers[l]["q"], layers[l]["kv"], ref))
    # all-F equals running each layer as its own DSA layer
    allf = [_layer(rng, L, H_I, d_I, H, d, True) for _ in range(3)]
    o_all, _, c_all = O.run_stack("FFF", allf, k)
    assert c_all == 3
    for l in range(3):
        ref = O.indexer_topk(allf[l]["q_I"], allf[l]["w"], allf[l]["k_I"], k)
        assert np.array_equal(o_all[l], O.sparse_attn(allf[l]["q"], allf[l]["kv"], ref))
    # '1'/'0' alphabet is the same pattern
    o10, _, c10 = O.run_stack("100100", layers, k)
    assert c10 == 2 and all(np.array_equal(a, b) for a, b in zip(o10, outs))
    with pytest.raises(O.NoCachedIndices):
        O.run_stack("SF", layers[1:3], k)
    with pytest.raises(ValueError):
        O.run_stack("FX", layers[:2], k)


def test_stack_quarter_of_indexers_kept():
    """[Abstract]: keeping one indexer in four removes 75% of indexer calls."""
    rng = np.random.default_rng(9)
    pattern = "FSSS" * 4
    layers = [_layer(rng, 8, 2, 4, 1, 4, c == "F") for c in pattern]
    _, _, calls = O.run_stack(pattern, layers, 4)
    assert calls == 4 and 1 - calls / len(pattern) == 0.75


def test_decode_step_equals_prefill_row():
    """Decode at seq_len = p+1 reproduces row p of a prefill over the same p+1 tokens."""
    rng = np.random.default_rng(10)
    L, H_I, d_I, H, d, k, B = 30, 3, 8, 2, 8, 5, 3
    pattern = "FSFS"
    seqs = [[_layer(rng, L, H_I, d_I, H, d, c == "F") for c in pattern] for _ in range(B)]
    seq_len = [L, 17, 1]
    dec_layers = []
    for l, c in enumerate(pattern):
        lay = {"q": np.stack([seqs[b][l]["q"][seq_len[b] - 1] for b in range(B)]),
               "kv": np.stack([seqs[b][l]["kv"] for b in range(B)])}
        if c == "F":
            lay.update(q_I=np.stack([seqs[b][l]["q_I"][seq_len[b] - 1] for b in range(B)]),
                       w=np.stack([seqs[b][l]["w"][seq_len[b] - 1] for b in range(B)]),
                       k_I=np.stack([seqs[b][l]["k_I"] for b in range(B)]))
        dec_layers.append(lay)
    outs, idxs, calls = O.decode_step(pattern, dec_layers, seq_len, k)
    assert calls == 2
    for b in range(B):
        n = seq_len[b]
        pre = [{key: v[:n] for key, v in lay.items()} for lay in seqs[b]]
        o_pre, used_pre, _ = O.run_stack(pattern, pre, k)
        for l in range(len(pattern)):
            assert np.array_equal(idxs[l][b], used_pre[l][n - 1])
            np.testing.assert_allclose(outs[l][b], o_pre[l][n - 1], rtol=0, atol=0)
    assert idxs[0][2].tolist() == [0, -1, -1, -1, -1]              # one visible key


def test_jaccard_example():
    """[Skill, Step 1] Jaccard of top-k sets: {1,2,3} vs {2,3,4} -> 2/4."""
    a = np.array([[1, 2, 3, -1]])
    b = np.array([[4, 3, 2, -1]])
    assert abs(O.jaccard_rows(a, b)[0] - 0.5) < 1e-7


def test_attention_extreme_logits_stay_finite():
    """Closed form at logits near +-1000: softmax is shift invariant per head, so a head whose
    logits are all very negative still gets weights e/(1+e), 1/(1+e) for a logit gap of 1."""
    d = 2
    kv = np.zeros((2, 2, d))
    kv[0, 0] = [1.0, 0.0]
    kv[1, 0] = [0.0, 1.0]
    kv[0, 1] = [1.0, 0.0]
    kv[1, 1] = [0.0, 1.0]
    q = np.array([[1000.0, 999.0], [-1000.0, -1001.0]])
    out = O.sparse_attn_row(q, kv, np.array([0, 1], dtype=np.int32), 1.0)
    e = math.e
    np.testing.assert_allclose(out, [[e / (1 + e), 1 / (1 + e)]] * 2, rtol=1e-13)


# ------------------------------------------------- distillation loss (fwd) --

def test_distill_two_entry_closed_form():
    """Closed form: one served layer, one head, two selected keys.  The target
    is a logistic pair sigma(delta), the indexer distribution sigma(eps), and
    KL = p0 ln(p0/r0) + p1 ln(p1/r1) (natural log), written out by hand."""
    d = 4
    q = np.array([[0.5, -1.0, 2.0, 0.25]])                   # [H=1, d]
    kv = np.zeros((3, 2, d))
    kv[0, 0] = [1.0, 0.0, 0.5, -2.0]
    kv[2, 0] = [-0.5, 1.0, 1.0, 4.0]
    idx = np.array([2, -1, 0], dtype=np.int32)               # entries: key 2 first, a hole, key 0
    scale = 1.0 / math.sqrt(d)
    I_t = np.array([3.0, 99.0, 1.25])                        # scores of keys 0..2 (key 1 unselected)
    dot0 = float(q[0] @ kv[0, 0]); dot2 = float(q[0] @ kv[2, 0])
    p_key2 = 1.0 / (1.0 + math.exp(-scale * (dot2 - dot0)))
    r_key2 = 1.0 / (1.0 + math.exp(-(1.25 - 3.0)))
    want = p_key2 * math.log(p_key2 / r_key2) + (1 - p_key2) * math.log((1 - p_key2) / (1 - r_key2))
    got = O.distill_kl_row(I_t, [q], [kv], idx, scale)
    assert abs(got - want) < 1e-12
    p = O.served_attention_row([q], [kv], idx, scale)
    assert abs(p[0] - p_key2) < 1e-12 and abs(p.sum() - 1.0) < 1e-12


def test_distill_gibbs_and_library_kl():
    """Gibbs' inequality (KL >= 0, = 0 iff the distributions agree) and torch's
    kl_div (a separate implementation of the same divergence)."""
    rng = np.random.default_rng(7)
    H, d, Lk, k = 3, 8, 40, 12
    qs = [rng.normal(size=(H, d)) for _ in range(3)]
    kvs = [rng.normal(size=(Lk, 2, d)) for _ in range(3)]
    idx = np.full(k, -1, dtype=np.int32)
    idx[:9] = rng.permutation(Lk)[:9]
    scale = 0.3
    I_t = rng.normal(size=Lk) * 4
    kl = O.distill_kl_row(I_t, qs, kvs, idx, scale)
    assert kl > 0
    p = O.served_attention_row(qs, kvs, idx, scale)
    sel = idx[idx >= 0]
    log_r = torch.log_softmax(torch.from_numpy(I_t[sel]), dim=0)
    lib = torch.nn.functional.kl_div(log_r, torch.from_numpy(p), reduction="sum").item()
    assert abs(kl - lib) < 1e-10
    matched = np.full(Lk, -50.0)
    matched[sel] = np.log(p) + 7.0                           # indexer distribution == target
    assert abs(O.distill_kl_row(matched, qs, kvs, idx, scale)) < 1e-12


def test_distill_invariances():
    """Shifting every indexer score leaves the loss alone; so do permuting the
    entries, moving the -1 holes, and serving the same layer twice; scaling the
    logits changes it."""
    rng = np.random.default_rng(11)
    H, d, Lk = 2, 6, 30
    q = rng.normal(size=(H, d)); kv = rng.normal(size=(Lk, 2, d))
    q2 = rng.normal(size=(H, d)); kv2 = rng.normal(size=(Lk, 2, d))
    sel = rng.permutation(Lk)[:10].astype(np.int32)
    idx = np.concatenate([sel[:4], [-1, -1], sel[4:]]).astype(np.int32)
    I_t = rng.normal(size=Lk) * 3
    base = O.distill_kl_row(I_t, [q, q2], [kv, kv2], idx, 0.4)
    assert abs(O.distill_kl_row(I_t + 123.0, [q, q2], [kv, kv2], idx, 0.4) - base) < 1e-9
    perm = np.concatenate([sel[::-1], [-1, -1]]).astype(np.int32)
    assert abs(O.distill_kl_row(I_t, [q, q2], [kv, kv2], perm, 0.4) - base) < 1e-12
    one = O.served_attention_row([q], [kv], idx, 0.4)
    twice = O.served_attention_row([q, q], [kv, kv], idx, 0.4)
    assert np.allclose(one, twice, atol=1e-15)
    both = O.served_attention_row([q, q2], [kv, kv2], idx, 0.4)
    assert np.allclose(both, 0.5 * (one + O.served_attention_row([q2], [kv2], idx, 0.4)), atol=1e-15)
    assert abs(O.distill_kl_row(2.0 * I_t, [q, q2], [kv, kv2], idx, 0.4) - base) > 1e-3


def test_distill_dense_case_is_causal_softmax_attention_weights():
    """Every visible key selected: the target is the head-mean of the causal
    softmax(Q K^T / sqrt(d)) rows, computed here with torch's masked softmax."""
    rng = np.random.default_rng(3)
    L, H, d, H_I, d_I = 9, 2, 4, 2, 3
    q = rng.normal(size=(L, H, d)); kv = rng.normal(size=(L, 2, d))
    q_I = rng.normal(size=(L, H_I, d_I)); w = rng.uniform(size=(L, H_I)); k_I = rng.normal(size=(L, d_I))
    idx = np.full((L, L), -1, dtype=np.int32)
    for t in range(L):
        idx[t, : t + 1] = np.arange(t + 1)
    Q = torch.from_numpy(q).permute(1, 0, 2)                 # [H, L, d]
    K = torch.from_numpy(kv[:, 0]).expand(H, L, d)
    att = (Q @ K.transpose(1, 2)) / math.sqrt(d)
    att = att.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
    target = torch.softmax(att, dim=-1).mean(0).numpy()       # [L, L]
    y = np.einsum("thc,sc->ths", q_I, k_I)
    I_full = np.einsum("th,ths->ts", w, np.maximum(y, 0.0))
    for t in range(L):
        p = O.served_attention_row([q[t]], [kv], idx[t], 1 / math.sqrt(d))
        assert np.allclose(p, target[t, : t + 1], atol=1e-12)
    kl = O.distill_kl(q_I, w, k_I, idx, [q], [kv])
    for t in range(L):
        r = np.exp(I_full[t, : t + 1] - I_full[t, : t + 1].max())
        r /= r.sum()
        want = float(np.sum(target[t, : t + 1] * np.log(target[t, : t + 1] / r)))
        assert abs(kl[t] - want) < 1e-10


# ------------------------------------------------------ dynamic refresh --

def test_probe_rows_end_at_the_last_query():
    assert O.probe_rows(10, 4).tolist() == [1, 5, 9]
    assert O.probe_rows(8, 1).tolist() == list(range(8))
    assert O.probe_rows(5, 64).tolist() == [4]


def _dyn_layers(L=12, H_I=2, d_I=3, H=1, d=4, seed=0, n=3):
    rng = np.random.default_rng(seed)
    return [dict(q=rng.normal(size=(L, H, d)), kv=rng.normal(size=(L, 2, d)),
                 q_I=rng.normal(size=(L, H_I, d_I)), w=rng.uniform(size=(L, H_I)), k_I=rng.normal(size=(L, d_I)))
            for _ in range(n)]


def test_dynamic_refresh_limits_are_the_static_patterns():
    """tau = 0 never refreshes (the static pattern); tau > 1 always refreshes
    (every layer runs its own indexer, as an all-F stack)."""
    lay = _dyn_layers()
    k = 4
    o_s, u_s, _ = O.run_stack("FSS", lay, k)
    o_f, u_f, _ = O.run_stack("FFF", lay, k)
    o0, u0, r0, rec0 = O.run_stack_dynamic("FSS", lay, k, stride=3, tau=0.0)
    assert not r0.any() and all(np.array_equal(a, b) for a, b in zip(u0, u_s))
    assert all(np.array_equal(a, b) for a, b in zip(o0, o_s))
    o1, u1, r1, rec1 = O.run_stack_dynamic("FSS", lay, k, stride=3, tau=1.01)
    assert r1.tolist() == [False, True, True] and all(np.array_equal(a, b) for a, b in zip(u1, u_f))
    assert np.isnan(rec1[0]) and np.all((rec1[1:] >= 0) & (rec1[1:] <= 1))


def test_dynamic_refresh_recall_by_hand():
    """The pooled recall, counted by hand: an S layer whose indexer inputs are
    the F layer's has recall exactly 1 and never refreshes below tau = 1; one
    whose scores reverse the order has recall counted from explicit sets."""
    lay = _dyn_layers(n=2)
    k, L = 4, 12
    same = [lay[0], dict(lay[1], q_I=lay[0]["q_I"], w=lay[0]["w"], k_I=lay[0]["k_I"])]
    _, _, ref, rec = O.run_stack_dynamic("FS", same, k, stride=5, tau=1.0)
    assert rec[1] == 1.0 and not ref[1]
    _, _, ref, rec = O.run_stack_dynamic("FS", same, k, stride=5, tau=1.0 + 1e-12)
    assert ref[1]
    cache = O.indexer_topk(lay[0]["q_I"], lay[0]["w"], lay[0]["k_I"], k)
    hit = own = 0
    for t in (1, 6, 11):                                     # probe rows for L = 12, stride 5
        sc = [float(lay[1]["w"][t] @ np.maximum(lay[1]["q_I"][t] @ lay[1]["k_I"][s], 0)) for s in range(t + 1)]
        order = sorted(range(t + 1), key=lambda s: (-np.float32(sc[s]), s))[:k]
        hit += len(set(order) & set(int(x) for x in cache[t] if x >= 0))
        own += len(order)
    _, _, _, rec = O.run_stack_dynamic("FS", lay, k, stride=5, tau=0.0)
    assert rec[1] == hit / own


def test_dynamic_refresh_probe_uses_absolute_positions():
    """Queries continuing a cached prefix (pos0 > 0): the probe scores query t at its
    absolute position pos0 + t, over keys 0..pos0 + t, exactly as the F layer did.  An S
    layer whose indexer inputs are the F layer's therefore still has recall exactly 1."""
    L, pos0, k = 12, 7, 4
    rng = np.random.default_rng(3)
    f = dict(q=rng.normal(size=(L, 1, 4)), kv=rng.normal(size=(pos0 + L, 2, 4)), q_I=rng.normal(size=(L, 2, 3)),
             w=rng.uniform(size=(L, 2)), k_I=rng.normal(size=(pos0 + L, 3)))
    _, used, ref, rec = O.run_stack_dynamic("FS", [f, dict(f)], k, stride=5, tau=1.0, pos0=pos0)
    assert rec[1] == 1.0 and not ref[1]
    assert np.array_equal(used[1], O.indexer_topk(f["q_I"], f["w"], f["k_I"], k, pos0))
