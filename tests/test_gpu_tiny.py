"""GPU parity on the tiny stack (B=1, L=512, 'FSSS', H_I=4, d_I=32, k=64, H=4, d=64):
small-integer inputs make every fp32 score exact, so scores and idx must equal the
oracle bit for bit, and attention must be within 1e-2 of fp64."""
import numpy as np
import pytest
import torch

import oracle as O
import dsa_lightning_indexer_scores_amd as ic
from dsa_lightning_indexer_scores_amd import synth
from parity_helpers import ATTN_TOL, attn_rel_err, dec, summary

pytestmark = pytest.mark.gpu
CFG = synth.WORKLOADS["tiny"]


@pytest.fixture(scope="module")
def stack():
    cpu = synth.prefill_stack(CFG, device="cpu")
    gpu = [{k: v.cuda() for k, v in lay.items()} for lay in cpu]
    ref = [{k: dec(v)[0] for k, v in lay.items()} for lay in cpu]           # batch 0, float64
    return cpu, gpu, ref


def test_scores_bit_exact(stack):
    _, gpu, ref = stack
    sc = ic.indexer_scores(gpu[0]["q_I"], gpu[0]["w"], gpu[0]["k_I"]).cpu().numpy()[0]
    rows = O.indexer_scores(ref[0]["q_I"], ref[0]["w"], ref[0]["k_I"])
    for t, r in enumerate(rows):
        assert np.array_equal(sc[t, : t + 1].astype(np.float64), r), f"row {t}"


def test_idx_bit_exact_and_chunk_invariant(stack):
    _, gpu, ref = stack
    want = O.indexer_topk(ref[0]["q_I"], ref[0]["w"], ref[0]["k_I"], CFG.k)
    for chunk in (0, 512, 128, 16):
        got = ic.indexer_topk(gpu[0]["q_I"], gpu[0]["w"], gpu[0]["k_I"], CFG.k, chunk=chunk).cpu().numpy()[0]
        assert np.array_equal(got, want), f"chunk={chunk}"
    assert got[0].tolist() == [0] + [-1] * (CFG.k - 1)


def test_stack_matches_oracle(stack):
    _, gpu, ref = stack
    outs, idx_cache, st = ic.run_stack(CFG.pattern, gpu, CFG.k)
    torch.cuda.synchronize()
    assert st["indexer_calls"] == CFG.pattern.count("F") == 1 and st["attn_calls"] == 4
    o_ref, used, calls = O.run_stack(CFG.pattern, ref, CFG.k)
    assert calls == 1
    assert np.array_equal(idx_cache.cpu().numpy()[0], used[-1])
    errs = [attn_rel_err(dec(outs[l])[0], o_ref[l]) for l in range(4)]
    summary("tiny stack attention", {"max_rel_err": max(errs)})
    assert max(errs) <= ATTN_TOL


def test_all_f_equals_per_layer_and_s_reuse(stack):
    _, gpu, _ = stack
    full = [dict(gpu[0], q=l["q"], kv=l["kv"]) for l in gpu]               # every layer gets layer 0's indexer
    outs_f, _, st = ic.run_stack("FFFF", full, CFG.k)
    assert st["indexer_calls"] == 4
    outs_s, _, _ = ic.run_stack("FSSS", gpu, CFG.k)
    idx0 = ic.indexer_topk(gpu[0]["q_I"], gpu[0]["w"], gpu[0]["k_I"], CFG.k)
    for l in range(4):
        alone = ic.sparse_attn(gpu[l]["q"], gpu[l]["kv"], idx0)
        assert torch.equal(outs_s[l], alone)                                # S layer == attention with F's idx
        assert torch.equal(outs_f[l], alone)                                # all-F == per-layer DSA
    outs_10, _, st10 = ic.run_stack("1000", gpu, CFG.k)
    assert st10["indexer_calls"] == 1 and all(torch.equal(a, b) for a, b in zip(outs_10, outs_s))


def test_s_first_is_an_error(stack):
    _, gpu, _ = stack
    with pytest.raises(ic.NoCachedIndices):
        ic.run_stack("SFSS", gpu, CFG.k)


def test_deterministic(stack):
    _, gpu, _ = stack
    a, ia, _ = ic.run_stack(CFG.pattern, gpu, CFG.k)
    b, ib, _ = ic.run_stack(CFG.pattern, gpu, CFG.k)
    assert torch.equal(ia, ib) and all(torch.equal(x, y) for x, y in zip(a, b))


def test_k_at_least_visible_selects_all_and_matches_dense(stack):
    """k >= L: every causal key is selected and sparse attention is dense causal attention."""
    _, gpu, ref = stack
    L = CFG.L
    small = {k: v[:, :L] for k, v in gpu[0].items()}
    idx = ic.indexer_topk(small["q_I"], small["w"], small["k_I"], 1024).cpu().numpy()[0]
    for t in (0, 1, 100, L - 1):
        assert idx[t, : t + 1].tolist() == list(range(t + 1)) and np.all(idx[t, t + 1:] == -1)
    out = ic.sparse_attn(gpu[1]["q"], gpu[1]["kv"], torch.from_numpy(idx)[None].cuda())
    q = torch.from_numpy(ref[1]["q"]).permute(1, 0, 2)[None]
    H = q.shape[1]
    kk = torch.from_numpy(ref[1]["kv"][:, 0]).expand(H, L, CFG.d)[None]
    vv = torch.from_numpy(ref[1]["kv"][:, 1]).expand(H, L, CFG.d)[None]
    dense = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, is_causal=True)[0].permute(1, 0, 2).numpy()
    assert attn_rel_err(dec(out)[0], dense) <= ATTN_TOL
