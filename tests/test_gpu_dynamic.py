"""GPU parity of drift-triggered dynamic refresh (ic_run_stack_dynamic).

An S layer that brings its own indexer inputs probes the cache on every
probe_stride-th query: it counts hit = sum |cached & own top-k| against own =
sum |own top-k| and re-indexes the whole sequence when hit < tau * own.  On
integer inputs every score is exact, so the probe's top-k, the counts, the
decisions, the recall (hit / own rounded to fp32) and every idx row must equal
the oracle exactly; attention outputs are held to the attention tolerance.
"""
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
    # every layer keeps its indexer inputs, so every S layer can probe and refresh
    cpu = synth.prefill_stack(CFG, device="cpu", pattern="FFFF")
    gpu = [{k: v.cuda() for k, v in lay.items()} for lay in cpu]
    ref = [{k: dec(v)[0] for k, v in lay.items()} for lay in cpu]
    return gpu, ref


def test_limits_equal_the_static_stacks(stack):
    gpu, _ = stack
    o_s, i_s, _ = ic.run_stack("FSSS", gpu, CFG.k)
    o_f, i_f, _ = ic.run_stack("FFFF", gpu, CFG.k)
    o0, i0, st0, r0, rec0 = ic.run_stack_dynamic("FSSS", gpu, CFG.k, probe_stride=16, tau=0.0)
    assert torch.equal(i0, i_s) and all(torch.equal(a, b) for a, b in zip(o0, o_s))
    assert r0[:, 0].tolist() == [-1, 0, 0, 0] and st0["indexer_calls"] == 1
    o1, i1, _, r1, rec1 = ic.run_stack_dynamic("FSSS", gpu, CFG.k, probe_stride=16, tau=1.01)
    assert torch.equal(i1, i_f) and all(torch.equal(a, b) for a, b in zip(o1, o_f))
    assert r1[:, 0].tolist() == [-1, 1, 1, 1]
    assert torch.isnan(rec0[0, 0]) and torch.all((rec0[1:] >= 0) & (rec0[1:] <= 1))


@pytest.mark.parametrize("stride", [1, 7, 64, 1000])
def test_decisions_recall_and_outputs_match_oracle(stack, stride):
    gpu, ref = stack
    _, _, _, rec0 = O.run_stack_dynamic("FSSS", ref, CFG.k, stride, 0.0)
    tau = float(np.median(rec0[1:]))                                      # mixed decisions
    outs, idx_cache, _, refreshed, recall = ic.run_stack_dynamic("FSSS", gpu, CFG.k, probe_stride=stride, tau=tau)
    torch.cuda.synchronize()
    o_ref, used, ref_refreshed, ref_recall = O.run_stack_dynamic("FSSS", ref, CFG.k, stride, tau)
    got_ref = refreshed.cpu().numpy()[:, 0]
    assert got_ref[0] == -1 and np.array_equal(got_ref[1:] == 1, ref_refreshed[1:])
    assert np.array_equal(recall.cpu().numpy()[1:, 0], ref_recall[1:].astype(np.float32))
    assert np.array_equal(idx_cache.cpu().numpy()[0], used[-1])
    errs = [attn_rel_err(dec(outs[l])[0], o_ref[l]) for l in range(4)]
    summary(f"dynamic stride={stride} tau={tau:.4f}", {"refreshed": got_ref.tolist(), "max_rel_err": max(errs)})
    assert max(errs) <= ATTN_TOL


def test_batch_and_cached_prefix(stack):
    """B = 2 sequences continuing a 100-token prefix: decisions are per sequence."""
    cpu = synth.prefill_stack(CFG, device="cpu", pattern="FFFF", B=2)
    p0 = 100
    gpu = []
    for lay in cpu:
        g = {k: v.cuda() for k, v in lay.items()}
        for key in ("q", "q_I", "w"):
            g[key] = g[key][:, p0:].contiguous()
        gpu.append(g)
    _, _, _, r0, rec0 = ic.run_stack_dynamic("FSSS", gpu, CFG.k, probe_stride=9, tau=0.0, pos0=p0)
    tau = float(np.median(rec0.cpu().numpy()[1:]))
    outs, idx_cache, _, refreshed, recall = ic.run_stack_dynamic("FSSS", gpu, CFG.k, probe_stride=9, tau=tau,
                                                                 pos0=p0)
    torch.cuda.synchronize()
    for b in range(2):
        ref = [{k: dec(v)[b] for k, v in lay.items()} for lay in cpu]
        for lay in ref:
            for key in ("q", "q_I", "w"):
                lay[key] = lay[key][p0:]
        o_ref, used, ref_refreshed, ref_recall = O.run_stack_dynamic("FSSS", ref, CFG.k, 9, tau, pos0=p0)
        assert np.array_equal(refreshed.cpu().numpy()[1:, b] == 1, ref_refreshed[1:])
        assert np.array_equal(recall.cpu().numpy()[1:, b], ref_recall[1:].astype(np.float32))
        assert np.array_equal(idx_cache.cpu().numpy()[b], used[-1])
        assert max(attn_rel_err(dec(outs[l])[b], o_ref[l]) for l in range(4)) <= ATTN_TOL


def test_s_layers_without_indexer_never_probe(stack):
    gpu, _ = stack
    plain = [gpu[0]] + [{k: v for k, v in l.items() if k in ("q", "kv")} for l in gpu[1:]]
    o_s, i_s, _ = ic.run_stack("FSSS", plain, CFG.k)
    o, i, _, refreshed, recall = ic.run_stack_dynamic("FSSS", plain, CFG.k, probe_stride=4, tau=1.5)
    assert torch.equal(i, i_s) and all(torch.equal(a, b) for a, b in zip(o, o_s))
    assert refreshed[:, 0].tolist() == [-1, -1, -1, -1] and torch.all(torch.isnan(recall))
