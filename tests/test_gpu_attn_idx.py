"""GPU parity of the sparse attention on idx rows that no top-k would write:
-1 entries anywhere in a row (single holes, whole 32-entry steps, everything but
the first or the last entry), unsorted entries and repeated entries.  The
attention contract only asks for at least one entry >= 0 per row and every
entry < Lk; a -1 is skipped wherever it sits and a repeated row counts twice.
Checked against the fp64 oracle fed the same idx, to the attention tolerance."""
import numpy as np
import pytest
import torch

import oracle as O
import dsa_lightning_indexer_scores_amd as ic
from parity_helpers import ATTN_TOL, attn_rel_err, dec, summary

pytestmark = pytest.mark.gpu


def idx_patterns(Lq: int, Lk: int, k: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    idx = np.full((Lq, k), -1, dtype=np.int32)
    for t in range(Lq):
        kind = t % 8
        row = rng.permutation(Lk)[:k].astype(np.int32)           # distinct, unsorted
        if kind == 0:                                            # only the last entry
            idx[t, k - 1] = row[0]
        elif kind == 1:                                          # only the first entry
            idx[t, 0] = row[0]
        elif kind == 2:                                          # scattered holes
            keep = rng.random(k) < 0.6
            idx[t] = np.where(keep, row, -1)
            idx[t, rng.integers(k)] = row[0]
        elif kind == 3:                                          # whole steps of -1 in the middle
            idx[t] = row
            idx[t, 32:64] = -1
            idx[t, 96:128] = -1
        elif kind == 4:                                          # repeated entries
            idx[t] = rng.integers(0, 5, size=k)
        elif kind == 5:                                          # sorted, trailing -1 (top-k shape)
            n = 1 + t % k
            idx[t, :n] = np.sort(row[:n])
        else:                                                    # every entry a row, unsorted
            idx[t] = row
    return idx


@pytest.mark.parametrize("d,H,k", [(128, 16, 200), (128, 20, 256), (64, 4, 200), (64, 16, 160)])
def test_attention_any_idx_layout(d, H, k):
    torch.manual_seed(d * 1000 + H + k)
    Lq, Lk = 64, 700
    q = (torch.randn(1, Lq, H, d) * 0.5).to(torch.bfloat16).cuda()
    kv = (torch.randn(1, Lk, 2, d) * 0.5).to(torch.bfloat16).cuda()
    idx = idx_patterns(Lq, Lk, k, seed=d + H + k)
    out = ic.sparse_attn(q, kv, torch.from_numpy(idx)[None].cuda())
    torch.cuda.synchronize()
    ref = O.sparse_attn(dec(q)[0], dec(kv)[0], idx)
    err = attn_rel_err(dec(out)[0], ref)
    summary(f"attention idx layouts d={d} H={H} k={k}", {"max_rel_err": err})
    assert err <= ATTN_TOL


@pytest.mark.parametrize("k", [1, 33, 257, 520, 4096])
def test_attention_idx_ring_boundaries(k):
    """The prefill kernel reads each idx row in 256-entry chunks and runs 32-entry steps:
    k = 1 (one partial step), 33 (one entry into a second step), 257 (one entry into a
    second chunk), 520 (three chunks, ragged) and 4096 (the largest k, sixteen chunks),
    with the same idx layouts as above."""
    torch.manual_seed(k)
    H, d = 16, 128
    Lq, Lk = (16, 4200) if k == 4096 else (48, max(700, k + 64))
    q = (torch.randn(1, Lq, H, d) * 0.5).to(torch.bfloat16).cuda()
    kv = (torch.randn(1, Lk, 2, d) * 0.5).to(torch.bfloat16).cuda()
    idx = idx_patterns(Lq, Lk, k, seed=k)
    if k < 2:                                                    # the layouts need room for holes
        idx = np.random.default_rng(k).integers(0, Lk, size=(Lq, k)).astype(np.int32)
    out = ic.sparse_attn(q, kv, torch.from_numpy(idx)[None].cuda())
    torch.cuda.synchronize()
    ref = O.sparse_attn(dec(q)[0], dec(kv)[0], idx)
    err = attn_rel_err(dec(out)[0], ref)
    summary(f"attention ring boundaries k={k}", {"max_rel_err": err})
    assert err <= ATTN_TOL


@pytest.mark.parametrize("d", [128, 64])
def test_rows_without_a_valid_entry_give_zero(d):
    """A row whose entries are all -1 or all >= Lk has nothing to attend to: its output
    vectors are zero (finite), and the other rows are unaffected."""
    torch.manual_seed(d)
    Lq, Lk, H, k = 40, 300, 16, 96
    q = (torch.randn(1, Lq, H, d) * 0.5).to(torch.bfloat16).cuda()
    kv = (torch.randn(1, Lk, 2, d) * 0.5).to(torch.bfloat16).cuda()
    idx = idx_patterns(Lq, Lk, k, seed=d)
    empty = [0, 7, 13, 39]
    idx[[0, 13]] = -1
    idx[7] = Lk + np.arange(k)                                   # past the KV rows
    idx[39, :] = -1
    idx[39, 5] = Lk                                              # one entry, out of range
    out = ic.sparse_attn(q, kv, torch.from_numpy(idx)[None].cuda())
    torch.cuda.synchronize()
    got = dec(out)[0]
    assert np.all(got[empty] == 0.0)
    keep = [t for t in range(Lq) if t not in empty]
    ref = O.sparse_attn(dec(q)[0][keep], dec(kv)[0], idx[keep])
    assert attn_rel_err(got[keep], ref) <= ATTN_TOL


def test_attention_largest_head_count():
    """H = 4096 (the largest the boundary accepts): 256 head groups per query, each its own
    wave, against the oracle on every query and head."""
    torch.manual_seed(4096)
    Lq, Lk, H, d, k = 4, 300, 4096, 64, 96
    q = (torch.randn(1, Lq, H, d) * 0.5).to(torch.bfloat16).cuda()
    kv = (torch.randn(1, Lk, 2, d) * 0.5).to(torch.bfloat16).cuda()
    idx = idx_patterns(Lq, Lk, k, seed=7)
    out = ic.sparse_attn(q, kv, torch.from_numpy(idx)[None].cuda())
    torch.cuda.synchronize()
    ref = O.sparse_attn(dec(q)[0], dec(kv)[0], idx)
    err = attn_rel_err(dec(out)[0], ref)
    summary("attention H=4096", {"max_rel_err": err})
    assert err <= ATTN_TOL


def test_attention_at_the_largest_kv_capacity():
    """Lk = 2^23 - 1 rows of 512 bytes (d = 128): the last row ends 512 bytes below 4 GiB,
    the limit of the gather kernels' 32-bit row offsets.  Prefill (the last 8 queries) and
    decode (split-K) attention over rows at both ends of the range, against the oracle on
    the gathered rows."""
    Lk, H, d, k, Lq = (1 << 23) - 1, 16, 128, 96, 8
    g = torch.Generator(device="cuda").manual_seed(23)
    kv = torch.empty((1, Lk, 2, d), dtype=torch.bfloat16, device="cuda")
    step = 1 << 20
    for r0 in range(0, Lk, step):                     # bounded temporaries
        n = min(step, Lk - r0)
        kv[0, r0:r0 + n] = (torch.randn((n, 2, d), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    q = (torch.randn((1, Lq, H, d), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    rng = np.random.default_rng(23)
    idx = np.empty((Lq, k), dtype=np.int32)
    for t in range(Lq):
        top = rng.choice(np.arange(Lk - 2000, Lk), size=k // 2, replace=False)
        low = rng.choice(np.arange(0, 2000), size=k // 4, replace=False)
        mid = rng.integers(0, Lk, size=k - k // 2 - k // 4)
        idx[t] = np.sort(np.concatenate([low, mid, top]))
    idx[0, -1] = Lk - 1                               # the very last row
    idx_gpu = torch.from_numpy(idx).cuda()
    out = ic.sparse_attn(q, kv, idx_gpu[None])
    dq = ic.decode_attn(q[0, -1:].reshape(1, 1, H, d).contiguous(), kv, idx_gpu[-1:].reshape(1, 1, k).contiguous())
    torch.cuda.synchronize()
    worst = 0.0
    for t in range(Lq):
        rows = kv[0, idx_gpu[t].long()]               # the selected rows only
        ref = O.sparse_attn_row(dec(q)[0, t], dec(rows), np.arange(k, dtype=np.int32), 1.0 / np.sqrt(d))
        worst = max(worst, attn_rel_err(dec(out)[0, t], ref))
        if t == Lq - 1:
            worst = max(worst, attn_rel_err(dec(dq)[0, 0], ref))
    del kv
    summary("attention at Lk = 2^23 - 1", {"max_rel_err": worst})
    assert worst <= ATTN_TOL
