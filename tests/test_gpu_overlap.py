"""GPU cross-layer overlap diagnostic (agent skill page, Step 1) against the oracle's
Jaccard and brute-force set counts: random sorted rows with padding, empty, identical
and disjoint rows, k = 1 and k = 4096, and the F layers of a real stack."""
import numpy as np
import pytest
import torch

import oracle as O
import dsa_lightning_indexer_scores_amd as ic
from dsa_lightning_indexer_scores_amd import synth

pytestmark = pytest.mark.gpu


def _rows(rng, rows, k, universe):
    """Ascending rows of distinct positions, each of random length 0..k, -1 padded."""
    out = np.full((rows, k), -1, dtype=np.int32)
    for r in range(rows):
        n = int(rng.integers(0, k + 1))
        out[r, :n] = np.sort(rng.choice(universe, size=n, replace=False))
    return out


def _check(a: np.ndarray, b: np.ndarray):
    inter, jac, rec, means = ic.index_overlap(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda())
    inter, jac, rec, means = inter.cpu().numpy(), jac.cpu().numpy(), rec.cpu().numpy(), means.cpu().numpy()
    want_i = np.array([len(set(x[x >= 0]) & set(y[y >= 0])) for x, y in zip(a, b)])
    nb = (b >= 0).sum(1)
    assert np.array_equal(inter, want_i)
    want_j = O.jaccard_rows(a, b)
    assert np.allclose(jac, want_j, rtol=2e-7, atol=1e-7)
    want_r = np.where(nb > 0, want_i / np.maximum(nb, 1), 0.0)
    assert np.allclose(rec, want_r, rtol=2e-7, atol=1e-7)
    assert abs(means[0] - want_j.mean()) <= 1e-5 and abs(means[1] - want_r.mean()) <= 1e-5


@pytest.mark.parametrize("k,universe", [(1, 3), (64, 100), (300, 2000), (2048, 4096), (4096, 9000)])
def test_overlap_random_rows(k, universe):
    rng = np.random.default_rng(k)
    rows = 257
    a = _rows(rng, rows, k, universe)
    b = _rows(rng, rows, k, universe)
    b[0] = a[0]                                       # identical
    a[1] = -1                                         # A empty
    b[2] = -1                                         # B empty
    a[3] = -1
    b[3] = -1                                         # both empty
    _check(a, b)


def test_overlap_disjoint_and_nested():
    k = 128
    a = np.full((3, k), -1, dtype=np.int32)
    b = np.full((3, k), -1, dtype=np.int32)
    a[0, :64] = np.arange(0, 128, 2)
    b[0, :64] = np.arange(1, 129, 2)                  # disjoint: 0
    a[1, :128] = np.arange(128)
    b[1, :32] = np.arange(0, 128, 4)                  # B inside A: recall 1, Jaccard 1/4
    a[2, :5] = [3, 9, 10, 50, 70]
    b[2, :4] = [9, 11, 50, 71]
    _check(a, b)


def test_overlap_of_stack_layers():
    """Two F layers of the tiny stack: the GPU's idx (bit-exact with the oracle on integer
    inputs) compared layer against layer."""
    cfg = synth.WORKLOADS["tiny"]
    layers = synth.prefill_stack(cfg, device="cuda", pattern="FF")
    idx = [ic.indexer_topk(l["q_I"], l["w"], l["k_I"], cfg.k) for l in layers]
    _check(idx[0].cpu().numpy()[0], idx[1].cpu().numpy()[0])


def test_overlap_matrix_of_four_layers():
    """The all-pairs heatmap over four F layers of the tiny stack (bit-exact idx on integer
    inputs): every entry against the oracle's Jaccard and set counts, the diagonal 1."""
    cfg = synth.WORKLOADS["tiny"]
    layers = synth.prefill_stack(cfg, device="cuda", pattern="FFFF")
    idx = [ic.indexer_topk(l["q_I"], l["w"], l["k_I"], cfg.k) for l in layers]
    J, R = ic.overlap_matrix(idx)
    cpu = [i.cpu().numpy()[0] for i in idx]
    for a in range(4):
        for b in range(4):
            want_j = O.jaccard_rows(cpu[a], cpu[b]).mean()
            sets = [(set(x[x >= 0]), set(y[y >= 0])) for x, y in zip(cpu[a], cpu[b])]
            want_r = np.mean([len(sa & sb) / len(sb) for sa, sb in sets])
            assert abs(J[a, b] - want_j) <= 1e-5 and abs(R[a, b] - want_r) <= 1e-5, (a, b)
    assert np.allclose(np.diag(J), 1.0, atol=1e-6) and np.allclose(J, J.T, atol=1e-6)
    text = ic.format_heatmap(J, [f"L{l}" for l in range(4)])
    assert text.count("\n") == 4 and "L3" in text
