"""GPU parity at moderate sizes the oracle finishes in seconds: several tiles, ragged
tails, batch > 1, a query offset (prefill continuing a cached prefix), both indexer
dtypes, and decode with ragged sequence lengths."""
import numpy as np
import pytest
import torch

import oracle as O
import dsa_lightning_indexer_scores_amd as ic
from dsa_lightning_indexer_scores_amd import synth
from parity_helpers import ATTN_TOL, attn_rel_err, check_topk_row, dec, gpu_score_rows, summary

pytestmark = pytest.mark.gpu


def _rand_layer(B, Lq, Lk, H_I, d_I, H, d, dtype, dist, seed, full=True):
    g = torch.Generator().manual_seed(seed)

    def vals(shape, dim):
        if dist == "int3":
            return torch.randint(-3, 4, shape, generator=g).float()
        return torch.randn(shape, generator=g) / (dim ** 0.5 if dist == "gauss_scaled" else 1.0)

    lay = {"q": synth.encode(vals((B, Lq, H, d), d), "bf16"), "kv": synth.encode(vals((B, Lk, 2, d), d), "bf16")}
    if full:
        lay["q_I"] = synth.encode(vals((B, Lq, H_I, d_I), d_I), dtype)
        lay["k_I"] = synth.encode(vals((B, Lk, d_I), d_I), dtype)
        lay["w"] = (torch.randint(0, 4, (B, Lq, H_I), generator=g).float() if dist == "int3"
                    else torch.rand((B, Lq, H_I), generator=g))
    return lay


CASES = [
    # B, Lq, pos0, H_I, d_I, k, H, d, dtype, dist, chunk
    (2, 1000, 0, 64, 128, 300, 16, 128, "bf16", "int3", 256),
    (1, 777, 2001, 64, 128, 256, 16, 128, "fp8", "gauss", 0),
    (1, 1500, 0, 20, 64, 100, 20, 64, "bf16", "gauss_scaled", 512),
    (1, 1203, 0, 64, 128, 2048, 16, 128, "fp8", "gauss", 400),
    (1, 640, 0, 7, 32, 64, 5, 128, "fp8", "int3", 0),
    # a single indexer head (the score is then a masked GEMM), both dtypes, bit-exact idx
    (1, 900, 100, 1, 64, 128, 16, 64, "fp8", "int3", 0),
    (1, 500, 0, 1, 32, 50, 3, 64, "bf16", "int3", 128),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}_L{c[1]}_p{c[2]}_{c[8]}_{c[9]}_k{c[5]}")
def test_stack_fs_vs_oracle(case):
    B, Lq, pos0, H_I, d_I, k, H, d, dtype, dist, chunk = case
    Lk = pos0 + Lq
    layers = [_rand_layer(B, Lq, Lk, H_I, d_I, H, d, dtype, dist, 100 + i, full=(c == "F"))
              for i, c in enumerate("FS")]
    gpu = [{kk: v.cuda() for kk, v in lay.items()} for lay in layers]
    outs, idx_cache, st = ic.run_stack("FS", gpu, k, chunk=chunk, pos0=pos0)
    torch.cuda.synchronize()
    assert st["indexer_calls"] == 1 and st["attn_calls"] == 2
    idx = idx_cache.cpu().numpy()
    n_cert = n_rows = 0
    ovl = []
    worst = 0.0
    for b in range(B):
        f = {kk: dec(v[b]) for kk, v in layers[0].items()}
        g = {kk: v[b:b + 1] for kk, v in gpu[0].items()}
        sc = gpu_score_rows(g["q_I"], g["w"], g["k_I"], range(Lq), chunk or 4096, pos0)
        for t in range(Lq):
            c, o, _ = check_topk_row(idx[b, t], f["q_I"][t], f["w"][t], f["k_I"], pos0 + t, k, H_I, d_I,
                                     gpu_scores=sc[t])
            n_cert += c
            n_rows += 1
            ovl.append(o)
        if dist == "int3":
            want = O.indexer_topk(f["q_I"], f["w"], f["k_I"], k, pos0)
            assert np.array_equal(idx[b], want)
        for l in range(2):
            ref = O.sparse_attn(dec(layers[l]["q"][b]), dec(layers[l]["kv"][b]), idx[b])
            worst = max(worst, attn_rel_err(dec(outs[l][b]), ref))
    summary(f"stack FS {case}", {"certified": f"{n_cert}/{n_rows}", "mean_overlap": np.mean(ovl),
                                 "attn_max_rel_err": worst})
    assert np.mean(ovl) >= 0.99
    assert worst <= ATTN_TOL


def test_chunk_size_invariance_fp8():
    lay = _rand_layer(1, 2500, 2500, 64, 128, 0, 0, "fp8", "gauss", 7)
    g = {kk: v.cuda() for kk, v in lay.items() if kk in ("q_I", "w", "k_I")}
    base = ic.indexer_topk(g["q_I"], g["w"], g["k_I"], 512, chunk=4096)
    for chunk in (16, 1008, 2496):
        assert torch.equal(ic.indexer_topk(g["q_I"], g["w"], g["k_I"], 512, chunk=chunk), base), chunk


def test_scores_match_oracle_within_bound_fp8():
    lay = _rand_layer(1, 700, 700, 64, 128, 0, 0, "fp8", "gauss", 8)
    g = {kk: v.cuda() for kk, v in lay.items() if kk in ("q_I", "w", "k_I")}
    sc = ic.indexer_scores(g["q_I"], g["w"], g["k_I"]).cpu().numpy()[0].astype(np.float64)
    f = {kk: dec(v[0]) for kk, v in lay.items() if kk in ("q_I", "w", "k_I")}
    from parity_helpers import error_bound
    worst = 0.0
    for t in range(0, 700, 13):
        ex = O.indexer_scores_row(f["q_I"][t], f["w"][t], f["k_I"], t)
        E = error_bound(f["q_I"][t], f["w"][t], f["k_I"], t + 1, 64, 128)
        assert np.all(np.abs(sc[t, : t + 1] - ex) <= E + 1e-30)
        worst = max(worst, float((np.abs(sc[t, : t + 1] - ex) / np.maximum(E, 1e-30)).max()))
    summary("fp8 scores vs exact", {"max_err_over_bound": worst})


# Split-K decode attention: k = 256 gives 8 splits (2 partials), k = 520 gives 16
# (17 tiles, the last one ragged), and k = 4096 gives 128 splits whose 32 partials,
# most of them empty (every row has fewer than k keys), take the looped combine.
@pytest.mark.parametrize("k", [256, 520, 4096])
@pytest.mark.parametrize("dtype,dist", [("bf16", "int3"), ("fp8", "gauss")])
def test_decode_ragged_vs_oracle_and_prefill(dtype, dist, k):
    B, cap, H_I, d_I, H, d = 3, 1100, 64, 128, 16, 128
    seq_len = [1100, 333, 1]
    pattern = "FSSF"
    caches = [_rand_layer(B, 1, cap, H_I, d_I, H, d, dtype, dist, 300 + i, full=(c == "F"))
              for i, c in enumerate(pattern)]
    layers = []
    for lay in caches:
        one = {"q": lay["q"], "kv": lay["kv"]}
        if "q_I" in lay:
            one.update(q_I=lay["q_I"], w=lay["w"], k_I=lay["k_I"])
        layers.append(one)
    gpu = [{kk: v.cuda() for kk, v in lay.items()} for lay in layers]
    sl = torch.tensor(seq_len, dtype=torch.int32, device="cuda")
    outs, idx_cache, st = ic.decode_step(pattern, gpu, sl, k)
    torch.cuda.synchronize()
    assert st["indexer_calls"] == 2 and st["attn_calls"] == 4
    # oracle decode (float64 decoded inputs)
    ref_layers = []
    for lay in layers:
        r = {"q": dec(lay["q"])[:, 0], "kv": dec(lay["kv"])}
        if "q_I" in lay:
            r.update(q_I=dec(lay["q_I"])[:, 0], w=dec(lay["w"])[:, 0], k_I=dec(lay["k_I"]))
        ref_layers.append(r)
    o_ref, idx_ref, calls = O.decode_step(pattern, ref_layers, seq_len, k)
    assert calls == 2
    gidx = idx_cache.cpu().numpy()[:, 0]
    for b in range(B):
        p = seq_len[b] - 1
        if dist == "int3":
            assert np.array_equal(gidx[b], idx_ref[-1][b])
        else:
            check_topk_row(gidx[b], ref_layers[3]["q_I"][b], ref_layers[3]["w"][b], ref_layers[3]["k_I"][b], p, k,
                           H_I, d_I)
    # attention of the last two layers with the GPU's idx (layer 3's indexer feeds layer 3)
    ref3 = np.stack([O.sparse_attn_row(ref_layers[3]["q"][b], ref_layers[3]["kv"][b], gidx[b], 1 / np.sqrt(d))
                     for b in range(B)])
    assert attn_rel_err(dec(outs[3])[:, 0], ref3) <= ATTN_TOL
    if dist == "int3":
        for l in range(4):
            assert attn_rel_err(dec(outs[l])[:, 0], o_ref[l]) <= ATTN_TOL
    # decode == last row of a prefill over the same tokens (GPU against GPU)
    b = 1
    n = seq_len[b]
    f = gpu[0]
    q_pre = torch.zeros((1, n, H_I, d_I), dtype=f["q_I"].dtype, device="cuda")
    w_pre = torch.zeros((1, n, H_I), device="cuda")
    q_pre[0, n - 1] = f["q_I"][b, 0]
    w_pre[0, n - 1] = f["w"][b, 0]
    pre = ic.indexer_topk(q_pre, w_pre, f["k_I"][b:b + 1, :n].contiguous(), k)
    _, idx_f0, _ = ic.decode_step("F", [gpu[0]], sl, k)
    assert torch.equal(pre[0, n - 1], idx_f0[b, 0])


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_single_token_prompt_and_single_head(dtype):
    """The smallest shapes: a one-token prompt (Lq = Lk = 1, so idx = [0, -1, ...]) and
    one attention head (fifteen empty lanes in its head group), in prefill and in decode."""
    H_I, d_I, H, d, k = 1, 32, 1, 64, 64
    layers = [_rand_layer(1, 1, 1, H_I, d_I, H, d, dtype, "int3", 500 + i, full=(c == "F")) for i, c in enumerate("FS")]
    gpu = [{kk: v.cuda() for kk, v in lay.items()} for lay in layers]
    outs, idx_cache, _ = ic.run_stack("FS", gpu, k)
    torch.cuda.synchronize()
    want = np.full(k, -1, dtype=np.int32)
    want[0] = 0
    assert np.array_equal(idx_cache.cpu().numpy()[0, 0], want)
    for l in range(2):
        # one visible key: the output is that key's V row exactly (bf16 in, bf16 out)
        v0 = layers[l]["kv"][0, 0, 1]
        assert torch.equal(outs[l][0, 0, 0].cpu(), v0), f"layer {l}"
    # decode: two sequences of one and three tokens, one head
    cap = 3
    caches = [_rand_layer(2, 1, cap, H_I, d_I, H, d, dtype, "int3", 520 + i, full=(c == "F")) for i, c in enumerate("FS")]
    gpu = [{kk: v.cuda() for kk, v in lay.items()} for lay in caches]
    seq_len = [1, 3]
    outs, idx_cache, _ = ic.decode_step("FS", gpu, torch.tensor(seq_len, dtype=torch.int32, device="cuda"), k)
    torch.cuda.synchronize()
    ref_layers = []
    for lay in caches:
        r = {"q": dec(lay["q"])[:, 0], "kv": dec(lay["kv"])}
        if "q_I" in lay:
            r.update(q_I=dec(lay["q_I"])[:, 0], w=dec(lay["w"])[:, 0], k_I=dec(lay["k_I"]))
        ref_layers.append(r)
    o_ref, idx_ref, _ = O.decode_step("FS", ref_layers, seq_len, k)
    assert np.array_equal(idx_cache.cpu().numpy()[:, 0], idx_ref[-1])
    for l in range(2):
        assert attn_rel_err(dec(outs[l])[:, 0], o_ref[l]) <= ATTN_TOL
