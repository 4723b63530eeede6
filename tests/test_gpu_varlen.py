"""Ragged batched prefill (ic_run_stack_varlen): sequences of different lengths, each
continuing its own cached prefix, packed in one call.  Checked bitwise against one
ic_run_stack per sequence (same kernels, B=1 with that sequence's pos0) and against the
oracle on integer inputs (idx bit-exact, attention within the 1e-2 bar)."""
import numpy as np
import pytest
import torch

import oracle as O
import dsa_lightning_indexer_scores_amd as ic
from dsa_lightning_indexer_scores_amd import synth
from parity_helpers import ATTN_TOL, attn_rel_err, dec

pytestmark = pytest.mark.gpu


def _gen(seed, shape, kind):
    g = torch.Generator().manual_seed(seed)
    if kind == "int":
        return torch.randint(-3, 4, shape, generator=g).float()
    if kind == "w":
        return torch.randint(0, 4, shape, generator=g).float()
    return torch.randn(shape, generator=g)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_varlen_matches_per_sequence_and_oracle(dtype):
    q_len = [300, 0, 1, 517, 64]
    pos0 = [0, 40, 700, 100, 1036]
    B, T, Lk = len(q_len), sum(q_len), 1100
    H_I, d_I, k, H, d = 64, 128, 256, 16, 128
    pattern = "FSSF"
    layers = []
    for l, c in enumerate(pattern):
        lay = {"q": synth.encode(_gen(10 * l, (T, H, d), "int"), "bf16").cuda(),
               "kv": synth.encode(_gen(10 * l + 1, (B, Lk, 2, d), "int"), "bf16").cuda()}
        if c == "F":
            lay["q_I"] = synth.encode(_gen(10 * l + 2, (T, H_I, d_I), "int"), dtype).cuda()
            lay["w"] = _gen(10 * l + 3, (T, H_I), "w").cuda()
            lay["k_I"] = synth.encode(_gen(10 * l + 4, (B, Lk, d_I), "int"), dtype).cuda()
        layers.append(lay)
    outs, idx, st = ic.run_stack_varlen(pattern, layers, k, q_len, pos0, chunk=256)
    torch.cuda.synchronize()
    assert st["indexer_calls"] == 2 and st["attn_calls"] == 4
    q0 = 0
    for b in range(B):
        n = q_len[b]
        if n == 0:
            continue
        one = []
        for lay in layers:
            o = {"q": lay["q"][q0:q0 + n].unsqueeze(0).contiguous(), "kv": lay["kv"][b:b + 1].contiguous()}
            if "q_I" in lay:
                o.update(q_I=lay["q_I"][q0:q0 + n].unsqueeze(0).contiguous(),
                         w=lay["w"][q0:q0 + n].unsqueeze(0).contiguous(), k_I=lay["k_I"][b:b + 1].contiguous())
            one.append(o)
        o1, i1, _ = ic.run_stack(pattern, one, k, chunk=256, pos0=pos0[b])
        torch.cuda.synchronize()
        assert torch.equal(i1[0], idx[q0:q0 + n]), f"sequence {b}: idx differs from its own run"
        for l in range(len(pattern)):
            assert torch.equal(o1[l][0], outs[l][q0:q0 + n]), f"sequence {b} layer {l}: output differs"
        if b in (0, 3):                            # oracle on two sequences (integer inputs: exact idx)
            ref = []
            for o in one:
                r = {"q": dec(o["q"])[0], "kv": dec(o["kv"])[0]}
                if "q_I" in o:
                    r.update(q_I=dec(o["q_I"])[0], w=dec(o["w"])[0], k_I=dec(o["k_I"])[0])
                ref.append(r)
            o_ref, idx_ref, calls = O.run_stack(pattern, ref, k, pos0=pos0[b])
            assert calls == 2
            assert np.array_equal(idx[q0:q0 + n].cpu().numpy(), idx_ref[-1])
            for l in range(len(pattern)):
                assert attn_rel_err(dec(outs[l][q0:q0 + n]), o_ref[l]) <= ATTN_TOL
        q0 += n


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_varlen_many_short_sequences_grouped(dtype):
    """70 sequences (more than one group of 64), lengths 0..200 with a few longer than the
    256-query chunk (those run alone), each continuing its own prefix: bitwise equal to one
    ic_run_stack per sequence on a sample of sequences, and to the oracle on two."""
    rng = np.random.default_rng(5)
    B = 70
    q_len = [int(x) for x in rng.integers(0, 200, size=B)]
    q_len[3], q_len[40], q_len[41] = 0, 300, 257          # empty; longer than the chunk
    Lk = 700
    pos0 = [int(rng.integers(0, Lk - n + 1)) for n in q_len]
    T = sum(q_len)
    H_I, d_I, k, H, d = 16, 64, 96, 4, 64
    pattern = "FSF"
    layers = []
    for l, c in enumerate(pattern):
        lay = {"q": synth.encode(_gen(50 * l, (T, H, d), "int"), "bf16").cuda(),
               "kv": synth.encode(_gen(50 * l + 1, (B, Lk, 2, d), "int"), "bf16").cuda()}
        if c == "F":
            lay["q_I"] = synth.encode(_gen(50 * l + 2, (T, H_I, d_I), "int"), dtype).cuda()
            lay["w"] = _gen(50 * l + 3, (T, H_I), "w").cuda()
            lay["k_I"] = synth.encode(_gen(50 * l + 4, (B, Lk, d_I), "int"), dtype).cuda()
        layers.append(lay)
    outs, idx, st = ic.run_stack_varlen(pattern, layers, k, q_len, pos0, chunk=256)
    torch.cuda.synchronize()
    assert st["indexer_calls"] == 2 and st["attn_calls"] == 3
    starts = np.concatenate([[0], np.cumsum(q_len)])
    for b in sorted({0, 1, 2, 4, 39, 40, 41, 42, 63, 64, 65, 69} | set(range(5, B, 9))):
        n, q0 = q_len[b], int(starts[b])
        if n == 0:
            continue
        one = []
        for lay in layers:
            o = {"q": lay["q"][q0:q0 + n].unsqueeze(0).contiguous(), "kv": lay["kv"][b:b + 1].contiguous()}
            if "q_I" in lay:
                o.update(q_I=lay["q_I"][q0:q0 + n].unsqueeze(0).contiguous(),
                         w=lay["w"][q0:q0 + n].unsqueeze(0).contiguous(), k_I=lay["k_I"][b:b + 1].contiguous())
            one.append(o)
        o1, i1, _ = ic.run_stack(pattern, one, k, chunk=256, pos0=pos0[b])
        torch.cuda.synchronize()
        assert torch.equal(i1[0], idx[q0:q0 + n]), f"sequence {b}: idx differs from its own run"
        for l in range(len(pattern)):
            assert torch.equal(o1[l][0], outs[l][q0:q0 + n]), f"sequence {b} layer {l}: output differs"
        if b in (2, 64):
            ref = []
            for o in one:
                r = {"q": dec(o["q"])[0], "kv": dec(o["kv"])[0]}
                if "q_I" in o:
                    r.update(q_I=dec(o["q_I"])[0], w=dec(o["w"])[0], k_I=dec(o["k_I"])[0])
                ref.append(r)
            o_ref, idx_ref, calls = O.run_stack(pattern, ref, k, pos0=pos0[b])
            assert np.array_equal(idx[q0:q0 + n].cpu().numpy(), idx_ref[-1])
            for l in range(len(pattern)):
                assert attn_rel_err(dec(outs[l][q0:q0 + n]), o_ref[l]) <= ATTN_TOL
