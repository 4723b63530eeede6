"""GPU parity of the multi-layer distillation loss (forward) against the fp64 oracle.

Per query t the loss is KL(p_t || r_t) in nats: p_t averages the attention
distributions of the served layers and heads over the query's selected
entries, r_t is the softmax of the F layer's indexer scores over the same
entries.  The GPU computes in fp32 (exp2/log2 domain) from the fp32 indexer
scores; the oracle decodes the same bytes and works in fp64.

Tolerance: |kl - ref| <= 2e-3 + 1e-4 |ref|.  The dominant error is the fp32
rounding of the indexer scores (|I| up to a few hundred, 2^-24 relative, so
~2e-5 absolute per score) entering ln r, plus fp32 exp/log and sums over up to
4096 entries; measured errors are an order of magnitude below the bound.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle as O
import dsa_lightning_indexer_scores_amd as ic
from dsa_lightning_indexer_scores_amd import synth
from parity_helpers import dec, sample_rows, summary

pytestmark = pytest.mark.gpu

ABS_TOL, REL_TOL = 2e-3, 1e-4


def _check(got, ref, what):
    err = np.abs(got - ref)
    bound = ABS_TOL + REL_TOL * np.abs(ref)
    summary(what, {"max_abs_err": float(err.max()), "max_ref": float(np.abs(ref).max()),
                   "worst_err_over_bound": float((err / bound).max())})
    assert np.all(err <= bound), f"{what}: worst {err.max()} at {int(err.argmax())}"


def _group(cfg, L, B=1, n_served=4, pattern=None):
    pattern = pattern or ("F" + "S" * (n_served - 1))
    lay = synth.prefill_stack(cfg, device="cuda", L=L, B=B, pattern=pattern)
    return lay


def test_tiny_group_matches_oracle():
    """tiny (integer inputs, bf16 indexer): the F layer serves itself and three S layers."""
    cfg = synth.WORKLOADS["tiny"]
    lay = _group(cfg, cfg.L)
    idx = ic.indexer_topk(lay[0]["q_I"], lay[0]["w"], lay[0]["k_I"], cfg.k)
    kl, mean = ic.distill_kl(lay[0]["q_I"], lay[0]["w"], lay[0]["k_I"], idx,
                             [l["q"] for l in lay], [l["kv"] for l in lay])
    torch.cuda.synchronize()
    ref_idx = O.indexer_topk(dec(lay[0]["q_I"])[0], dec(lay[0]["w"])[0], dec(lay[0]["k_I"])[0], cfg.k)
    assert np.array_equal(idx.cpu().numpy()[0], ref_idx)
    ref = O.distill_kl(dec(lay[0]["q_I"])[0], dec(lay[0]["w"])[0], dec(lay[0]["k_I"])[0], ref_idx,
                       [dec(l["q"])[0] for l in lay], [dec(l["kv"])[0] for l in lay])
    got = kl.cpu().numpy()[0]
    _check(got, ref, "distill tiny")
    assert abs(float(mean.item()) - float(np.mean(got.astype(np.float64)))) <= 1e-6 * max(1.0, abs(float(np.mean(got))))
    kl2, mean2 = ic.distill_kl(lay[0]["q_I"], lay[0]["w"], lay[0]["k_I"], idx,
                               [l["q"] for l in lay], [l["kv"] for l in lay])
    assert torch.equal(kl, kl2) and torch.equal(mean, mean2)                 # deterministic


@pytest.mark.parametrize("d,H,k,n_served,B,pos0", [(128, 16, 100, 2, 1, 0), (64, 20, 64, 3, 2, 37),
                                                   (128, 4, 256, 1, 1, 300)])
def test_shapes_holes_and_ragged(d, H, k, n_served, B, pos0):
    """Ragged k (not a multiple of 32), two head groups (H = 20), d = 64, B = 2,
    queries continuing a cached prefix, and idx rows with -1 holes, unsorted
    entries and entries past the visible keys (all ignored)."""
    torch.manual_seed(d + H + k)
    Lq, Lk, H_I, d_I = 96, 96 + pos0, 8, 64
    rng = np.random.default_rng(k)
    q_I = (torch.randn(B, Lq, H_I, d_I) * 0.3).to(torch.bfloat16).cuda()
    w = torch.rand(B, Lq, H_I).cuda()
    k_I = (torch.randn(B, Lk, d_I) * 0.3).to(torch.bfloat16).cuda()
    qs = [(torch.randn(B, Lq, H, d) * 0.5).to(torch.bfloat16).cuda() for _ in range(n_served)]
    kvs = [(torch.randn(B, Lk, 2, d) * 0.5).to(torch.bfloat16).cuda() for _ in range(n_served)]
    idx = np.full((B, Lq, k), -1, dtype=np.int32)
    for b in range(B):
        for t in range(Lq):
            vis = pos0 + t + 1
            m = min(k, vis)
            row = rng.permutation(vis)[:m].astype(np.int32)
            row[rng.random(m) < 0.2] = -1                                   # holes
            if m < k and t % 3 == 0:
                row = np.concatenate([row, [vis + 5] if vis + 5 < Lk else [-1]]).astype(np.int32)
            if not np.any(row >= 0):
                row[0] = t % vis
            idx[b, t, : row.shape[0]] = row
    kl, mean = ic.distill_kl(q_I, w, k_I, torch.from_numpy(idx).cuda(), qs, kvs, pos0=pos0, chunk=32)
    torch.cuda.synchronize()
    got = kl.cpu().numpy()
    for b in range(B):
        clean = idx[b].copy()
        for t in range(Lq):
            clean[t][clean[t] > pos0 + t] = -1                             # past the visible keys: ignored
        ref = O.distill_kl(dec(q_I)[b], dec(w)[b], dec(k_I)[b], clean, [dec(q)[b] for q in qs],
                           [dec(kv)[b] for kv in kvs], pos0=pos0)
        _check(got[b], ref, f"distill d={d} H={H} k={k} served={n_served} b={b}")
    assert abs(float(mean.item()) - float(got.astype(np.float64).mean())) <= 1e-6 * max(1.0, abs(float(got.mean())))


def test_dense_loss_when_every_visible_key_is_listed():
    """k >= L with every visible key listed: the dense form of the loss."""
    cfg = dataclasses.replace(synth.WORKLOADS["tiny"], L=256)
    lay = _group(cfg, 256, n_served=2)
    idx = ic.indexer_topk(lay[0]["q_I"], lay[0]["w"], lay[0]["k_I"], 256)
    assert np.all(idx.cpu().numpy()[0][np.triu_indices(256, 1)] == -1)     # every visible key, -1 after
    kl, _ = ic.distill_kl(lay[0]["q_I"], lay[0]["w"], lay[0]["k_I"], idx, [l["q"] for l in lay],
                          [l["kv"] for l in lay])
    ref = O.distill_kl(dec(lay[0]["q_I"])[0], dec(lay[0]["w"])[0], dec(lay[0]["k_I"])[0], idx.cpu().numpy()[0],
                       [dec(l["q"])[0] for l in lay], [dec(l["kv"])[0] for l in lay])
    _check(kl.cpu().numpy()[0], ref, "distill dense tiny")


def test_stack32k_first_group_sampled_rows():
    """Full size, in the configuration the benchmark times: stack32k's first F layer
    (fp8 indexer, k = 2048) serving itself and its three S layers, all 32768 queries,
    checked on sampled rows (chunk borders, first and last, random)."""
    cfg = synth.WORKLOADS["stack32k"]
    lay = _group(cfg, cfg.L)
    idx = ic.indexer_topk(lay[0]["q_I"], lay[0]["w"], lay[0]["k_I"], cfg.k, chunk=cfg.chunk)
    kl, mean = ic.distill_kl(lay[0]["q_I"], lay[0]["w"], lay[0]["k_I"], idx, [l["q"] for l in lay],
                             [l["kv"] for l in lay], chunk=cfg.chunk)
    torch.cuda.synchronize()
    got = kl.cpu().numpy()[0]
    assert np.all(np.isfinite(got)) and np.all(got >= -1e-3)
    rows = sample_rows(cfg.L, 10, seed=5)
    gidx = idx.cpu().numpy()[0]
    k_I = dec(lay[0]["k_I"])[0]
    kvs = [dec(l["kv"])[0] for l in lay]
    scale = 1.0 / math.sqrt(cfg.d)
    ref = []
    for t in rows:                                                        # decode only the sampled queries
        I_t = O.indexer_scores_row(dec(lay[0]["q_I"][0, t]), dec(lay[0]["w"][0, t]), k_I, int(t))
        ref.append(O.distill_kl_row(I_t, [dec(l["q"][0, t]) for l in lay], kvs, gidx[t], scale))
    _check(got[rows], np.array(ref), "distill stack32k sampled")
