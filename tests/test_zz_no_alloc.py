"""ic_decode_step_static, the decode step for callers that cannot allocate (no workspace:
the library's fixed per-GPU scratch array), against ic_decode_step with a workspace.
Both run the same kernels, so outputs and indices must be bitwise equal; two calls in a
row, the second on a smaller input, check that nothing depends on what the first left
in the shared array."""
import ctypes

import pytest
import torch

import dsa_lightning_indexer_scores_amd as ic
from dsa_lightning_indexer_scores_amd import synth

pytestmark = pytest.mark.gpu


def _decode_inputs(B, cap, H_I, d_I, H, d, dtype, pattern, seed):
    g = torch.Generator().manual_seed(seed)
    layers = []
    for c in pattern:
        lay = {"q": synth.encode(torch.randn((B, 1, H, d), generator=g), "bf16"),
               "kv": synth.encode(torch.randn((B, cap, 2, d), generator=g), "bf16")}
        if c == "F":
            lay["q_I"] = synth.encode(torch.randn((B, 1, H_I, d_I), generator=g), dtype)
            lay["k_I"] = synth.encode(torch.randn((B, cap, d_I), generator=g), dtype)
            lay["w"] = torch.randn((B, 1, H_I), generator=g)
        layers.append({kk: v.cuda() for kk, v in lay.items()})
    return layers


CALLS = [
    # B, cap, seq_len, H_I, d_I, H, d, k, dtype, pattern
    (4, 40000, [40000, 33000, 517, 1], 64, 128, 16, 128, 2048, "fp8", "FSSF"),   # segmented top-k, 32 splits
    (2, 900, [900, 77], 20, 64, 20, 64, 256, "bf16", "FS"),                      # smaller: fewer splits, 2 head groups
]


def test_static_scratch_matches_workspace_path_twice():
    for i, (B, cap, sl, H_I, d_I, H, d, k, dtype, pattern) in enumerate(CALLS):
        print(f"[no-alloc] call {i}: B={B} cap={cap} k={k} {dtype} {pattern}", flush=True)
        layers = _decode_inputs(B, cap, H_I, d_I, H, d, dtype, pattern, 900 + i)
        seq_len = torch.tensor(sl, dtype=torch.int32, device="cuda")
        shape = ic._stack_shape(pattern, layers, k, 0, 0)
        assert ic.workspace_size(shape, ic.IC_OP_DECODE_STEP) <= 32 << 20
        o_ws, i_ws, st_ws = ic.decode_step(pattern, layers, seq_len, k)
        o_st = [torch.full_like(l["q"], float("nan")) for l in layers]
        i_st = torch.full((B, 1, k), -7, dtype=torch.int32, device="cuda")
        o_st, i_st, st_st = ic.decode_step_static(pattern, layers, seq_len, k, outs=o_st, idx_cache=i_st)
        torch.cuda.synchronize()
        assert st_st == st_ws
        assert torch.equal(i_st, i_ws), f"call {i}: indices differ"
        for l in range(len(pattern)):
            assert torch.equal(o_st[l], o_ws[l]), f"call {i}: layer {l} output differs"


def test_static_scratch_rejects_oversized_shapes():
    shape = ic.make_shape(B=64, Lq=1, Lk=200000, k=2048, H=16, d=128, H_I=64, d_I=128, idx_dtype=ic.IC_FP8_E4M3)
    assert ic.workspace_size(shape, ic.IC_OP_DECODE_STEP) > 32 << 20
    fake = ctypes.c_void_p(0x1000)
    arr = (ic.Layer * 1)(ic.Layer(fake, fake, fake, fake, fake, fake))
    r = ic.lib().ic_decode_step_static(b"F", 1, arr, ctypes.byref(shape), fake, fake, None, None)
    assert r == ic.IC_ERR_WORKSPACE and "static scratch" in ic.last_error()


def test_static_scratch_under_graph_capture():
    """The static entry point captured in a HIP graph (outputs preallocated, so the capture
    records kernel launches only) and replayed with new queries, caches and lengths: every
    replay equals the workspace path called eagerly, bitwise."""
    B, cap, H_I, d_I, H, d, k, pattern = 2, 900, 20, 64, 20, 64, 256, "FS"
    layers = _decode_inputs(B, cap, H_I, d_I, H, d, "bf16", pattern, 950)
    seq_len = torch.tensor([900, 77], dtype=torch.int32, device="cuda")
    outs = [torch.empty_like(l["q"]) for l in layers]
    idx = torch.empty((B, 1, k), dtype=torch.int32, device="cuda")
    run = lambda: ic.decode_step_static(pattern, layers, seq_len, k, outs=outs, idx_cache=idx)
    run()                                   # the first call on a device looks up the scratch address
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    g = torch.Generator(device="cuda").manual_seed(5)
    for rep, lens in enumerate(([450, 899], [1, 600], [900, 900])):
        print(f"[no-alloc] graph replay {rep}: seq_len {lens}", flush=True)
        for lay in layers:
            for name in ("q", "kv", "q_I", "k_I", "w"):
                if name in lay:
                    lay[name].copy_(torch.randn(lay[name].shape, generator=g, device="cuda").to(lay[name].dtype))
        seq_len.copy_(torch.tensor(lens, dtype=torch.int32))
        graph.replay()
        torch.cuda.synchronize()
        got_o, got_i = [o.clone() for o in outs], idx.clone()
        ref_o, ref_i, _ = ic.decode_step(pattern, layers, seq_len, k)
        torch.cuda.synchronize()
        assert torch.equal(got_i, ref_i), f"replay {rep}: indices differ"
        for l in range(len(pattern)):
            assert torch.equal(got_o[l], ref_o[l]), f"replay {rep}: layer {l} output differs"
