"""Cache rows past the visible context are never used.

A KV or indexer-key cache may hold more rows than a call's context (the capacity that
decode steps will fill).  Those rows may hold anything, so here they hold poison: NaN in
every KV row, and indexer keys of 448 (the e4m3 maximum) in every channel, which would
outscore every real key if a query could see them.  Every output must still equal the
oracle's, which never reads those rows: idx bit-exact (small-integer inputs), attention
within the usual tolerance and finite.  Queries with fewer visible keys than k also carry
-1 padding in their idx rows, whose masked entries must not pick up a poisoned row
either."""
import numpy as np
import pytest
import torch

import oracle as O
import dsa_lightning_indexer_scores_amd as ic
from dsa_lightning_indexer_scores_amd import synth
from parity_helpers import ATTN_TOL, attn_rel_err, dec, summary

pytestmark = pytest.mark.gpu

POISON_KEY = 448.0


def _layer(B, Lq, Lk, n_ctx, H_I, d_I, H, d, dtype, seed, full):
    """Integer inputs in [-3, 3]; rows n_ctx[b].. of sequence b's caches poisoned."""
    g = torch.Generator().manual_seed(seed)

    def ri(shape):
        return torch.randint(-3, 4, shape, generator=g).float()

    kv = ri((B, Lk, 2, d))
    for b in range(B):
        kv[b, n_ctx[b]:] = float("nan")
    lay = {"q": synth.encode(ri((B, Lq, H, d)), "bf16"), "kv": kv.to(torch.bfloat16)}
    if full:
        k_I = ri((B, Lk, d_I))
        for b in range(B):
            k_I[b, n_ctx[b]:] = POISON_KEY
        lay["q_I"] = synth.encode(ri((B, Lq, H_I, d_I)), dtype)
        lay["k_I"] = synth.encode(k_I, dtype)
        lay["w"] = torch.randint(0, 4, (B, Lq, H_I), generator=g).float()
    return lay


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("B,Lq,pos0", [(2, 1, 0), (1, 5, 37), (2, 300, 1000)])
def test_prefill_ignores_rows_past_the_context(dtype, B, Lq, pos0):
    H_I, d_I, H, d, k, extra = 20, 64, 16, 128, 64, 64
    Lk = pos0 + Lq + extra
    n_ctx = [pos0 + Lq] * B
    layers = [_layer(B, Lq, Lk, n_ctx, H_I, d_I, H, d, dtype, 900 + i, full=(c == "F")) for i, c in enumerate("FS")]
    gpu = [{kk: v.cuda() for kk, v in lay.items()} for lay in layers]
    outs, idx_cache, st = ic.run_stack("FS", gpu, k, chunk=128, pos0=pos0)
    torch.cuda.synchronize()
    assert st["indexer_calls"] == 1
    idx = idx_cache.cpu().numpy()
    worst = 0.0
    for b in range(B):
        f = {kk: dec(v[b]) for kk, v in layers[0].items()}
        want = O.indexer_topk(f["q_I"], f["w"], f["k_I"], k, pos0)
        assert np.array_equal(idx[b], want), f"sequence {b}: idx differ from the oracle"
        for l in range(2):
            got = dec(outs[l][b])
            assert np.isfinite(got).all(), f"layer {l}, sequence {b}: non-finite output"
            ref = O.sparse_attn(dec(layers[l]["q"][b]), dec(layers[l]["kv"][b]), idx[b])
            worst = max(worst, attn_rel_err(got, ref))
    summary(f"capacity prefill {dtype} B{B} Lq{Lq} pos0{pos0}", {"attn_max_rel_err": worst})
    assert worst <= ATTN_TOL


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_decode_ignores_rows_past_the_sequence(dtype):
    B, cap, H_I, d_I, H, d, k = 3, 700, 64, 128, 16, 128, 128
    seq_len = [636, 100, 1]
    pattern = "FS"
    caches = [_layer(B, 1, cap, seq_len, H_I, d_I, H, d, dtype, 950 + i, full=(c == "F"))
              for i, c in enumerate(pattern)]
    gpu = [{kk: v.cuda() for kk, v in lay.items()} for lay in caches]
    sl = torch.tensor(seq_len, dtype=torch.int32, device="cuda")
    outs, idx_cache, st = ic.decode_step(pattern, gpu, sl, k)
    torch.cuda.synchronize()
    ref_layers = []
    for lay in caches:
        r = {"q": dec(lay["q"])[:, 0], "kv": dec(lay["kv"])}
        if "q_I" in lay:
            r.update(q_I=dec(lay["q_I"])[:, 0], w=dec(lay["w"])[:, 0], k_I=dec(lay["k_I"]))
        ref_layers.append(r)
    o_ref, idx_ref, calls = O.decode_step(pattern, ref_layers, seq_len, k)
    assert calls == 1
    gidx = idx_cache.cpu().numpy()[:, 0]
    assert np.array_equal(gidx, idx_ref[-1]), "decode idx differ from the oracle"
    for l in range(len(pattern)):
        got = dec(outs[l])[:, 0]
        assert np.isfinite(got).all(), f"layer {l}: non-finite output"
        assert attn_rel_err(got, o_ref[l]) <= ATTN_TOL


def test_attention_entries_outside_the_cache_are_skipped():
    """idx entries of -1, negative or >= Lk are skipped, here with the cache's last row NaN."""
    B, Lq, Lk, H, d, k = 1, 64, 300, 16, 128, 96
    rng = np.random.default_rng(31)
    lay = _layer(B, Lq, Lk, [Lk - 1], 1, 32, H, d, "bf16", 990, full=False)
    idx = np.sort(rng.choice(Lk - 1, size=(Lq, k)), axis=1).astype(np.int32)
    holes = rng.random((Lq, k))
    idx[holes < 0.1] = -1
    idx[(holes >= 0.1) & (holes < 0.15)] = Lk + 5
    idx[(holes >= 0.15) & (holes < 0.2)] = -7
    idx[0, :] = -1                                        # a row with no valid entry: zeros
    out = ic.sparse_attn(lay["q"].cuda(), lay["kv"].cuda(), torch.from_numpy(idx[None]).cuda())
    torch.cuda.synchronize()
    got = dec(out[0])
    assert np.isfinite(got).all()
    assert np.all(got[0] == 0.0)
    skipped = np.where((idx >= 0) & (idx < Lk), idx, -1)
    ref = O.sparse_attn(dec(lay["q"][0])[1:], dec(lay["kv"][0]), skipped[1:])
    assert attn_rel_err(got[1:], ref) <= ATTN_TOL


def test_distill_ignores_rows_past_the_context():
    """The distillation loss over the GPU's own top-k, plus entries naming poisoned rows
    (visible to no query), which are ignored like any entry outside the visible keys."""
    B, Lq, pos0, H_I, d_I, H, d, k, extra = 1, 160, 40, 8, 64, 16, 128, 48, 32
    Lk = pos0 + Lq + extra
    n_ctx = [pos0 + Lq]
    lay = [_layer(B, Lq, Lk, n_ctx, H_I, d_I, H, d, "bf16", 970 + j, full=(j == 0)) for j in range(3)]
    g = [{kk: v.cuda() for kk, v in l.items()} for l in lay]
    idx = ic.indexer_topk(g[0]["q_I"], g[0]["w"], g[0]["k_I"], k, pos0=pos0).cpu().numpy()
    idx[0, ::3, -1] = Lk - 1                             # a poisoned row, past every query's keys
    kl, _ = ic.distill_kl(g[0]["q_I"], g[0]["w"], g[0]["k_I"], torch.from_numpy(idx).cuda(),
                          [l["q"] for l in g], [l["kv"] for l in g], pos0=pos0, chunk=64)
    torch.cuda.synchronize()
    got = kl.cpu().numpy()[0]
    assert np.isfinite(got).all()
    clean = np.where(idx[0] >= n_ctx[0], -1, idx[0])
    ref = O.distill_kl(dec(lay[0]["q_I"])[0], dec(lay[0]["w"])[0], dec(lay[0]["k_I"])[0], clean,
                       [dec(l["q"])[0] for l in lay], [dec(l["kv"])[0] for l in lay], pos0=pos0)
    err = np.abs(got - ref)
    bound = 2e-3 + 1e-4 * np.abs(ref)
    summary("capacity distill", {"worst_err_over_bound": float((err / bound).max())})
    assert np.all(err <= bound)
