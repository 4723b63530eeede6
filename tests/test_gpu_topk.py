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


@pytest.mark.parametrize("n0", [4000, 4091, 6000, 8187, 12000, 20000, 40000, 70000])
def test_topk_long_rows(n0):
    """Rows on both sides of the LDS staging limit and of each block shape's key capacity
    (4096, 8192: the last row of n0 = 4091 and 8187 is exactly that long); k = 2048 as in
    the DSA configs."""
    rng = np.random.default_rng(n0)
    rows = 6
    m = np.abs(rng.standard_normal((rows, n0 + rows)).astype(np.float32)) * 30
    m[:, 5::7] = np.float32(31.0)                       # a heavy tie near the threshold
    _run(m, n0, 2048)


@pytest.mark.parametrize("n0", [6000, 20000, 30000, 40000])
def test_topk_long_rows_largest_k(n0):
    """The largest k (4096) in the many-row mode: rows held in registers by each block
    shape (512 x 16, 1024 x 24, 1024 x 32) and streamed rows, with the output staged in the
    histograms' LDS at its full size and a heavy tie near the threshold."""
    rng = np.random.default_rng(n0 + 1)
    rows = 5
    m = np.abs(rng.standard_normal((rows, n0 + rows)).astype(np.float32)) * 30
    m[:, 2::9] = np.float32(27.0)
    _run(m, n0, 4096)


@pytest.mark.parametrize("n_last,k,kind", [(8192, 2048, "random"), (16384, 2048, "ties"), (16384, 4096, "random"),
                                           (24576, 2048, "random"), (24576, 2048, "threshold_tie"),
                                           (32768, 2048, "ties"), (32768, 4096, "threshold_tie")])
def test_topk_many_rows(n_last, k, kind):
    """Launches of 1024 rows take the several-rows-per-CU shapes (512 x 16, 512 x 32,
    1024 x 24 held to 64 VGPRs, 512 x 64); the last row fills its shape exactly.  Every row
    against the oracle, with heavy integer ties, random scores, and ties straddling the
    k-th key."""
    rng = np.random.default_rng(n_last + k)
    rows = 1024
    first = n_last - rows + 1
    if kind == "ties":
        m = rng.integers(-3, 4, size=(rows, n_last)).astype(np.float32)
    elif kind == "random":
        m = (rng.standard_normal((rows, n_last)) * 50).astype(np.float32)
    else:
        m = np.abs(rng.standard_normal((rows, n_last)).astype(np.float32)) * 30
        m[:, 3::11] = np.float32(40.0)
    _run(m, first, k)


@pytest.mark.parametrize("n_last,kind", [(8192, "ties"), (16384, "random"), (24576, "threshold_tie"), (32768, "random")])
def test_topk_many_rows_unaligned(n_last, kind):
    """The same several-rows-per-CU shapes with an odd row stride (n_last + 1 floats), which
    takes their scalar-load variants; every row against the oracle."""
    rng = np.random.default_rng(n_last + 7)
    rows, k = 1024, 2048
    first = n_last - rows + 1
    if kind == "ties":
        m = rng.integers(-3, 4, size=(rows, n_last + 1)).astype(np.float32)
    elif kind == "random":
        m = (rng.standard_normal((rows, n_last + 1)) * 50).astype(np.float32)
    else:
        m = np.abs(rng.standard_normal((rows, n_last + 1)).astype(np.float32)) * 30
        m[:, 3::11] = np.float32(40.0)
    _run(m, first, k)


def test_topk_k_larger_than_rows():
    m = np.random.default_rng(1).standard_normal((8, 40)).astype(np.float32)
    _run(m, 10, 64)


def _run_seq(mat: np.ndarray, lens, k: int):
    """ic_topk_rows_seq, segmented and streamed, against the oracle on every row."""
    rows, stride = mat.shape
    sc = torch.from_numpy(mat).cuda()
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    seg = ic.topk_rows_seq(sc, sl, k).cpu().numpy()
    one = ic.topk_rows_seq(sc, sl, k, segmented=False).cpu().numpy()
    for r in range(rows):
        want = O.topk_row(mat[r, :lens[r]], k)
        assert np.array_equal(seg[r], want), f"segmented row {r} (n={lens[r]}, k={k})"
        assert np.array_equal(one[r], want), f"streamed row {r} (n={lens[r]}, k={k})"


@pytest.mark.parametrize("kind", ["ties", "zeros_signed", "random", "threshold_tie"])
def test_topk_rows_seq_long(kind):
    """Decode-shaped rows longer than one register block: the segmented path (segment
    top-k, then a select over the candidates) must equal the oracle, with ragged last
    segments, rows shorter than the longest (empty segments), and rows with n <= k."""
    rng = np.random.default_rng({"ties": 1, "zeros_signed": 2, "random": 3, "threshold_tie": 4}[kind])
    stride, k = 70001, 2048
    lens = [70001, 65600, 40000, 32769, 8193, 2048, 100, 1]
    rows = len(lens)
    if kind == "ties":
        m = rng.integers(-3, 4, size=(rows, stride)).astype(np.float32)
    elif kind == "zeros_signed":
        m = np.where(rng.random((rows, stride)) < 0.5, -0.0, 0.0).astype(np.float32)
        m[:, ::37] = 1.0
    elif kind == "random":
        m = (rng.standard_normal((rows, stride)) * 50).astype(np.float32)
    else:
        m = np.abs(rng.standard_normal((rows, stride)).astype(np.float32)) * 30
        m[:, 3::11] = np.float32(40.0)                    # ties straddling the k-th key
    _run_seq(m, lens, k)


@pytest.mark.parametrize("k", [1, 100, 4096])
def test_topk_rows_seq_k(k):
    rng = np.random.default_rng(k)
    lens = [50000, 33000, 4096, 4097]
    m = rng.integers(-20, 20, size=(len(lens), 50000)).astype(np.float32)
    _run_seq(m, lens, k)


@pytest.mark.parametrize("kind", ["random", "threshold_tie"])
def test_topk_multi_million_key_rows(kind):
    """Rows of about 4.2 million keys, streamed block by block through every pass, at the
    largest k; the last row ends in a ragged block."""
    rng = np.random.default_rng({"random": 5, "threshold_tie": 6}[kind])
    n0, rows = (1 << 22) + 3, 2
    if kind == "random":
        m = (rng.standard_normal((rows, n0 + rows)) * 50).astype(np.float32)
    else:
        m = np.abs(rng.standard_normal((rows, n0 + rows)).astype(np.float32)) * 30
        m[:, 3::11] = np.float32(120.0)               # ties straddling the k-th key
    _run(m, n0, 4096)


@pytest.mark.parametrize("n_last,kind", [(40000, "random"), (65536, "threshold_tie"), (40001, "random")])
def test_topk_many_streamed_rows(n_last, kind):
    """Launches of 1024 rows of 40K-64K keys stream 512-thread blocks, four rows per CU
    (an odd row stride, 40001, takes the unaligned scalar-load variant, two rows per CU);
    every 8th row, the first and the last are checked against the oracle."""
    rng = np.random.default_rng(n_last)
    rows, k = 1024, 2048
    first = n_last - rows + 1
    if kind == "random":
        m = (rng.standard_normal((rows, n_last)) * 50).astype(np.float32)
    else:
        m = np.abs(rng.standard_normal((rows, n_last)).astype(np.float32)) * 30
        m[:, 3::11] = np.float32(40.0)
    got = ic.topk_rows(torch.from_numpy(m).cuda(), first, k).cpu().numpy()
    for r in sorted(set(range(0, rows, 8)) | {rows - 1}):
        want = O.topk_row(m[r, :first + r], k)
        assert np.array_equal(got[r], want), f"row {r} (n={first + r})"
