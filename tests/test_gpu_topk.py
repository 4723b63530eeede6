"""GPU top-k on chosen score rows vs the oracle's brute-force stable sort, bit-exact:
ties, -0.0 against +0.0, all-equal rows, k >= n, negative scores, and rows long
enough to take the global-memory path."""
import numpy as np
import pytest
import torch

import oracle as O
import dsa_lightning_indexer_scores_amd as ic

pytestmark = pytest.mark.gpu


def _run(mat: np.ndarray, first_len: int, k: int):
    rows, stride = mat.shape
    got = ic.topk_rows(torch.from_numpy(mat).cuda(), first_len, k).cpu().numpy()
    for r in range(rows):
        n = first_len + r
        want = O.topk_row(mat[r, :n], k)
        assert np.array_equal(got[r], want), f"row {r} (n={n}, k={k})"


@pytest.mark.parametrize("kind", ["ties", "zeros_signed", "equal", "increasing", "decreasing", "negative", "random"])
@pytest.mark.parametrize("k", [1, 7, 64, 300])
def test_topk_rows_small(kind, k):
    rng = np.random.default_rng(hash((kind, k)) % 2**32)
    rows, first = 97, 200
    stride = first + rows
    if kind == "ties":
        m = rng.integers(-3, 4, size=(rows, stride)).astype(np.float32)
    elif kind == "zeros_signed":
        m = np.where(rng.random((rows, stride)) < 0.5, -0.0, 0.0).astype(np.float32)
        m[:, ::17] = 1.0
    elif kind == "equal":
        m = np.full((rows, stride), 2.5, np.float32)
    elif kind == "increasing":
        m = np.tile(np.arange(stride, dtype=np.float32), (rows, 1))
    elif kind == "decreasing":
        m = np.tile(-np.arange(stride, dtype=np.float32), (rows, 1))
    elif kind == "negative":
        m = -np.abs(rng.standard_normal((rows, stride))).astype(np.float32)
    else:
        m = (rng.standard_normal((rows, stride)) * 50).astype(np.float32)
    _run(m, first, k)


@pytest.mark.parametrize("n0", [4000, 20000, 40000, 70000])
def test_topk_long_rows(n0):
    """Rows on both sides of the LDS staging limit; k = 2048 as in the DSA configs."""
    rng = np.random.default_rng(n0)
    rows = 6
    m = np.abs(rng.standard_normal((rows, n0 + rows)).astype(np.float32)) * 30
    m[:, 5::7] = np.float32(31.0)                       # a heavy tie near the threshold
    _run(m, n0, 2048)


def test_topk_k_larger_than_rows():
    m = np.random.default_rng(1).standard_normal((8, 40)).astype(np.float32)
    _run(m, 10, 64)
