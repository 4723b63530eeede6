"""Shared helpers of the GPU parity tests: decoding inputs for the oracle, the
attention error metric and the margin certificate for floating-point top-k.

Tolerances (stated here once, used by every parity test):
  * integer / index outputs: bit-exact (idx rows, and fp32 scores whenever the
    inputs are small integers, where every partial sum is an exact integer);
  * attention: per output vector (query, head), max_c |o - ref| divided by
    max(max_c |ref|, 1e-6) must be <= 1e-2 against the fp64 oracle, fed the
    idx the GPU used;
  * top-k on non-integer inputs: a row is certified when the gap between the
    oracle's k-th and (k+1)-th float32 scores exceeds twice the fp32
    accumulation bound E = 2 (d_I + H_I) 2^-24 sum_j |w_j| sum_c |q_jc k_sc|
    (plus 2 ulp); certified rows must equal the oracle row exactly, every
    other row must be a valid top-k within that bound;
  * given the GPU's own fp32 scores of a row (from the launches its top-k
    ranked), every row is checked exactly in two stages: each score lies within
    E (plus the final fp32 rounding) of the oracle's exact score of that key,
    and the idx row equals the oracle's top-k of those fp32 scores bit for bit.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle as O
import dsa_lightning_indexer_scores_amd as ic
from dsa_lightning_indexer_scores_amd import synth

ATTN_TOL = 1e-2


def dec(t: torch.Tensor, dtype: str = None) -> np.ndarray:
    """A GPU/CPU input tensor -> float64 numpy, decoded by the oracle from its raw bytes."""
    if t.dtype == torch.bfloat16:
        return O.decode_bf16(synth.bits_u16(t))
    if t.dtype == torch.uint8:
        return O.decode_e4m3(synth.bits_u8(t))
    return t.detach().cpu().double().numpy()


def attn_rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max over (query, head) of max_c |o - ref| / max(max_c |ref|, 1e-6)."""
    err = np.abs(gpu - ref).max(axis=-1)
    scale = np.maximum(np.abs(ref).max(axis=-1), 1e-6)
    return float((err / scale).max())


def error_bound(q_I_t: np.ndarray, w_t: np.ndarray, k_I: np.ndarray, n: int, H_I: int, d_I: int) -> np.ndarray:
    absdot = np.abs(q_I_t) @ np.abs(k_I[:n]).T          # [H_I, n]
    return 2.0 * (d_I + H_I) * 2.0 ** -24 * (np.abs(w_t) @ absdot)


def check_topk_row(gpu_row: np.ndarray, q_I_t, w_t, k_I, p: int, k: int, H_I: int, d_I: int,
                   gpu_scores: np.ndarray = None):
    """Certify one row.  Returns (certified, overlap, exact_match); asserts validity, and
    with gpu_scores (the GPU's fp32 scores of the row's visible keys) the two-stage check."""
    exact = O.indexer_scores_row(q_I_t, w_t, k_I, p)
    n = p + 1
    if gpu_scores is not None:
        got = np.asarray(gpu_scores[:n], dtype=np.float32)
        tol = error_bound(q_I_t, w_t, k_I, n, H_I, d_I) + 2.0 ** -24 * np.abs(exact) + 1e-300
        bad = np.abs(got.astype(np.float64) - exact) > tol
        assert not bad.any(), f"row at p={p}: {int(bad.sum())} scores outside the fp32 bound"
        assert np.array_equal(gpu_row, O.topk_row(got, k)), \
            f"row at p={p}: idx differ from the oracle's top-k of the GPU's own scores"
    ref = O.topk_row(O.to_decision_precision(exact), k)
    m = min(k, n)
    sel = gpu_row[:m]
    assert np.all(gpu_row[m:] == -1), "padding must be -1"
    assert np.all(sel >= 0) and np.all(sel < n), "indices out of the visible range"
    assert np.all(np.diff(sel) > 0), "row must be strictly ascending"
    match = bool(np.array_equal(gpu_row, ref))
    overlap = len(set(sel.tolist()) & set(ref[:m].tolist())) / m
    if m == n:
        assert match
        return True, 1.0, True
    E = error_bound(q_I_t, w_t, k_I, n, H_I, d_I).max()
    v = np.sort(O.to_decision_precision(exact).astype(np.float64))[::-1]
    ulp = 2.0 * abs(np.spacing(np.float32(v[k - 1]))) if v[k - 1] != 0 else 0.0
    certified = (v[k - 1] - v[k]) > 2 * E + ulp
    if certified:
        assert match, f"certified row at p={p} differs from the oracle"
    mask = np.zeros(n, bool)
    mask[sel] = True
    slack = 2 * E + ulp + 1e-300
    if (~mask).any():
        assert exact[mask].min() >= exact[~mask].max() - slack, f"row at p={p} is not a valid top-k"
    return certified, overlap, match


def gpu_score_rows(q_I, w, k_I, rows, chunk: int, pos0: int = 0) -> dict:
    """The GPU's fp32 scores of sampled query rows of one sequence (B = 1), from the
    launches a chunked stack makes: each chunk's queries at their own positions against
    the keys up to the chunk's end.  Returns {row t: scores of keys 0 .. pos0 + t}."""
    L = q_I.shape[1]
    got = {}
    for c0 in range(0, L, chunk):
        sel = [int(t) for t in rows if c0 <= t < c0 + chunk]
        if not sel:
            continue
        nq = min(chunk, L - c0)
        sc = ic.indexer_scores(q_I[:, c0:c0 + nq], w[:, c0:c0 + nq], k_I, pos0=pos0 + c0)
        picked = sc[0, torch.as_tensor([t - c0 for t in sel], device=sc.device)].cpu().numpy()
        for t, r in zip(sel, picked):
            got[t] = r[:pos0 + t + 1]
        del sc
    return got


def sample_rows(L: int, n_random: int, seed: int, chunk: int = 4096) -> np.ndarray:
    """First rows, last rows, chunk borders and random rows."""
    rng = np.random.default_rng(seed)
    base = {0, 1, 2, 63, 64, L // 2, L - 2, L - 1}
    for c in range(chunk, L, chunk):
        base.update({c - 1, c})
    base.update(rng.integers(0, L, size=n_random).tolist())
    return np.array(sorted(x for x in base if 0 <= x < L))


def summary(name: str, stats: dict):
    print(f"[parity] {name}: " + ", ".join(f"{k}={v}" for k, v in stats.items()), flush=True)
