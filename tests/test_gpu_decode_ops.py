"""GPU parity of the decode step's kernels called one at a time: ic_decode_indexer_scores
(bit-exact fp32 scores on small-integer inputs, w of either sign, ragged sequence lengths)
and ic_decode_attn (the split-K decode attention with its fixed-order merge) on idx rows no
top-k would write (holes, unsorted and repeated entries, rows with no valid entry), against
the fp64 oracle; and both against what ic_decode_step computes with the same inputs,
bitwise."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import dsa_lightning_indexer_scores_amd as ic
from dsa_lightning_indexer_scores_amd import synth
from parity_helpers import ATTN_TOL, attn_rel_err, dec, summary

pytestmark = pytest.mark.gpu


def _int(shape, g, lo=-3):
    return torch.randint(lo, 4, shape, generator=g).float()


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
@pytest.mark.parametrize("H_I,d_I", [(64, 128), (20, 64), (1, 32), (40, 32), (16, 128), (5, 64)])
def test_decode_indexer_scores_bit_exact(dtype, H_I, d_I):
    g = torch.Generator().manual_seed(H_I * 7 + d_I)
    B, cap = 4, 3001
    seq_len = [3001, 1025, 64, 1]
    q_I = synth.encode(_int((B, 1, H_I, d_I), g), dtype).cuda()
    k_I = synth.encode(_int((B, cap, d_I), g), dtype).cuda()
    w = _int((B, 1, H_I), g).cuda()
    sl = torch.tensor(seq_len, dtype=torch.int32, device="cuda")
    sc = ic.decode_indexer_scores(q_I, w, k_I, sl).cpu().numpy().astype(np.float64)
    for b in range(B):
        want = O.indexer_scores_row(dec(q_I[b, 0]), dec(w[b, 0]), dec(k_I[b]), seq_len[b] - 1)
        assert np.array_equal(sc[b, : seq_len[b]], want), f"row {b}"


def _idx_rows(B, k, seq_len, cap, rng):
    idx = np.full((B, k), -1, dtype=np.int32)
    for b in range(B):
        n = seq_len[b]
        kind = b % 5
        row = rng.permutation(n)[: min(k, n)].astype(np.int32)
        if kind == 0:                                  # every entry a row, unsorted
            idx[b, : len(row)] = row
        elif kind == 1:                                # scattered holes
            keep = rng.random(len(row)) < 0.5
            idx[b, : len(row)] = np.where(keep, row, -1)
            idx[b, 0] = row[0]
        elif kind == 2:                                # repeated entries
            idx[b] = rng.integers(0, min(n, 7), size=k)
        elif kind == 3:                                # sorted with -1 padding (the top-k shape)
            idx[b, : len(row)] = np.sort(row)
        else:                                          # nothing valid (-1, or past the cache): zero output
            idx[b] = -1
            idx[b, k // 2] = cap + 5
    return idx


@pytest.mark.parametrize("k", [256, 520, 2048, 4096])
@pytest.mark.parametrize("H,d", [(16, 128), (20, 64)])
def test_decode_attn_vs_oracle(k, H, d):
    rng = np.random.default_rng(k + H + d)
    g = torch.Generator().manual_seed(k * 3 + H)
    B, cap = 5, 5000
    seq_len = [5000, 4100, 700, 2, 3000]
    q = synth.encode(torch.randn((B, 1, H, d), generator=g) * 0.5, "bf16").cuda()
    kv = synth.encode(torch.randn((B, cap, 2, d), generator=g) * 0.5, "bf16").cuda()
    idx = _idx_rows(B, k, seq_len, cap, rng)
    out = ic.decode_attn(q, kv, torch.from_numpy(idx)[:, None].cuda())
    torch.cuda.synchronize()
    got = dec(out)[:, 0]
    worst = 0.0
    for b in range(B):
        valid = idx[b][(idx[b] >= 0) & (idx[b] < cap)]
        if valid.size == 0:
            assert np.all(got[b] == 0.0), f"row {b} has no valid entry and must be zero"
            continue
        ref = O.sparse_attn_row(dec(q[b, 0]), dec(kv[b]), idx[b], 1.0 / np.sqrt(d))
        worst = max(worst, attn_rel_err(got[b], ref))
    summary(f"decode_attn k={k} H={H} d={d}", {"max_rel_err": worst})
    assert worst <= ATTN_TOL


def test_decode_ops_equal_decode_step():
    """One 'FS' decode step against the same work done call by call: decode indexer scores,
    segmented top-k of those rows, decode attention of both layers."""
    cfg = dataclasses.replace(synth.WORKLOADS["decode64k"], pattern="FS")
    B, N = 6, 40000
    caches = synth.decode_caches(cfg, device="cuda", N=N, B=B, steps=1)
    qs = synth.decode_queries(cfg, 0, device="cuda", B=B)
    layers = [dict(caches[l], **qs[l]) for l in range(2)]
    sl = torch.tensor([N + 1, N, 31000, 20000, 5, 1], dtype=torch.int32, device="cuda")
    outs, idx, _ = ic.decode_step("FS", layers, sl, cfg.k)
    sc = ic.decode_indexer_scores(layers[0]["q_I"], layers[0]["w"], layers[0]["k_I"], sl)
    idx2 = ic.topk_rows_seq(sc, sl, cfg.k, max_len=N + 1)
    assert torch.equal(idx2, idx[:, 0])
    for l in range(2):
        o = ic.decode_attn(layers[l]["q"], layers[l]["kv"], idx)
        assert torch.equal(o, outs[l]), f"layer {l}"


@pytest.mark.parametrize("B,H,d", [(96, 64, 128), (2, 4096, 64)])
def test_decode_attn_one_split_per_query(B, H, d):
    """With enough (sequence, head group) pairs the decode attention runs one wave per pair
    and no split-K merge (fewer than four splits per query): 96 sequences x 4 head groups,
    and the largest head count (4096 heads = 256 groups) with 2 sequences.  Against the
    oracle, with holes, repeated entries and an empty row among the idx rows."""
    rng = np.random.default_rng(B * 7 + H)
    g = torch.Generator().manual_seed(B + H)
    cap, k = 700, 160
    seq_len = [int(x) for x in rng.integers(1, cap + 1, size=B)]
    q = synth.encode(torch.randn((B, 1, H, d), generator=g) * 0.5, "bf16").cuda()
    kv = synth.encode(torch.randn((B, cap, 2, d), generator=g) * 0.5, "bf16").cuda()
    idx = _idx_rows(B, k, seq_len, cap, rng)
    out = ic.decode_attn(q, kv, torch.from_numpy(idx)[:, None].cuda())
    torch.cuda.synchronize()
    got = dec(out)[:, 0]
    qd, kvd = dec(q), dec(kv)
    worst = 0.0
    for b in range(B):
        valid = idx[b][(idx[b] >= 0) & (idx[b] < cap)]
        if valid.size == 0:
            assert np.all(got[b] == 0.0), f"row {b} has no valid entry and must be zero"
            continue
        ref = O.sparse_attn_row(qd[b, 0], kvd[b], idx[b], 1.0 / np.sqrt(d))
        worst = max(worst, attn_rel_err(got[b], ref))
    summary(f"decode_attn one split B={B} H={H} d={d}", {"max_rel_err": worst})
    assert worst <= ATTN_TOL


def test_decode_lengths_out_of_range_are_clamped():
    """seq_len values outside 1..Lk (0, negative, past the cache) come from device memory the
    host cannot check; the decode indexer and top-k clamp them to 1..Lk, never reading or
    writing past a row.  Scores and idx equal the oracle's at the clamped lengths."""
    g = torch.Generator().manual_seed(77)
    B, cap, H_I, d_I, k = 4, 3000, 16, 64, 256
    seq_len = [0, -7, cap + 50, 1500]
    clamped = [min(max(n, 1), cap) for n in seq_len]
    q_I = synth.encode(_int((B, 1, H_I, d_I), g), "fp8").cuda()
    k_I = synth.encode(_int((B, cap, d_I), g), "fp8").cuda()
    w = _int((B, 1, H_I), g).cuda()
    sl = torch.tensor(seq_len, dtype=torch.int32, device="cuda")
    sc = ic.decode_indexer_scores(q_I, w, k_I, sl)
    idx = ic.topk_rows_seq(sc, sl, k, max_len=cap)
    torch.cuda.synchronize()
    scn = sc.cpu().numpy().astype(np.float64)
    got = idx.cpu().numpy()
    for b in range(B):
        n = clamped[b]
        want = O.indexer_scores_row(dec(q_I[b, 0]), dec(w[b, 0]), dec(k_I[b]), n - 1)
        assert np.array_equal(scn[b, :n], want), f"row {b}"
        assert np.array_equal(got[b], O.topk_row(want.astype(np.float32), k)), f"row {b}"
