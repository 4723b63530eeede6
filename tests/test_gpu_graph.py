"""HIP graphs and streams: a decode step, a prefill stack (its side-stream tile work
included), a ragged batch and a stack with drift-triggered refresh (its decisions on the
device) captured in HIP graphs and replayed, every replay, with new inputs copied into the
static buffers and eager work in between, equal to the eager call; two prefill stacks in
flight at once on two caller streams, and from two host threads; and the one-tile workspace (every top-k on the
caller's stream) equal to the two-tile one.  All comparisons are bitwise."""
import pytest
import torch

import dsa_lightning_indexer_scores_amd as ic
from dsa_lightning_indexer_scores_amd import synth

pytestmark = pytest.mark.gpu


def test_decode_graph_replays_match_eager():
    B, cap, H_I, d_I, k, H, d = 4, 3000, 64, 128, 512, 16, 128
    pattern = "FSSF"
    g = torch.Generator(device="cuda").manual_seed(5)

    def rnd(*shape):
        return torch.randn(*shape, generator=g, device="cuda")

    caches = []
    for c in pattern:
        lay = {"kv": rnd(B, cap, 2, d).to(torch.bfloat16)}
        if c == "F":
            lay["k_I"] = synth.encode(rnd(B, cap, d_I), "fp8")
        caches.append(lay)

    def step_inputs(step):
        out = []
        for c in pattern:
            lay = {"q": rnd(B, 1, H, d).to(torch.bfloat16)}
            if c == "F":
                lay["q_I"] = synth.encode(rnd(B, 1, H_I, d_I), "fp8")
                lay["w"] = torch.rand(B, 1, H_I, generator=g, device="cuda")
            out.append(lay)
        seq = torch.tensor([cap - 3 + step % 3, 700 + step, 1 + step, 2048], dtype=torch.int32, device="cuda")
        return out, seq

    static_in, static_seq = step_inputs(0)
    layers = [dict(caches[l], **static_in[l]) for l in range(len(pattern))]
    outs = [torch.empty_like(l["q"]) for l in layers]
    idx = torch.empty((B, 1, k), dtype=torch.int32, device="cuda")
    shape = ic._stack_shape(pattern, layers, k, 0, 0)
    ws = torch.empty(ic.workspace_size(shape, ic.IC_OP_DECODE_STEP), dtype=torch.uint8, device="cuda")
    ic.decode_step(pattern, layers, static_seq, k, outs=outs, idx_cache=idx, ws=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ic.decode_step(pattern, layers, static_seq, k, outs=outs, idx_cache=idx, ws=ws)
    for step in range(1, 5):
        new_in, new_seq = step_inputs(step)
        for l in range(len(pattern)):
            for name, t in new_in[l].items():
                layers[l][name].copy_(t)
        static_seq.copy_(new_seq)
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        got_idx = idx.clone()
        # eager reference on separate buffers, same inputs
        ref_outs, ref_idx, _ = ic.decode_step(pattern, layers, static_seq, k)
        torch.cuda.synchronize()
        assert torch.equal(got_idx, ref_idx), f"replay {step}: idx differs"
        for l in range(len(pattern)):
            assert torch.equal(got[l], ref_outs[l]), f"replay {step}: layer {l} differs"


def test_prefill_stack_graph_replays_match_eager():
    """run_stack with several score tiles per F layer (its attention runs tile by tile on a
    side stream) captured in a graph: every replay with new inputs equals the eager call."""
    cfg = synth.WORKLOADS["tiny"]
    pattern, chunk = "FSFS", 96                                  # 512 queries: six tiles, the last ragged
    layers = synth.prefill_stack(cfg, device="cuda", pattern=pattern)
    outs = [torch.empty_like(l["q"]) for l in layers]
    idx = torch.empty((1, cfg.L, cfg.k), dtype=torch.int32, device="cuda")
    shape = ic._stack_shape(pattern, layers, cfg.k, chunk, 0)
    ws = torch.empty(ic.workspace_size(shape, ic.IC_OP_RUN_STACK), dtype=torch.uint8, device="cuda")
    ic.run_stack(pattern, layers, cfg.k, chunk=chunk, outs=outs, idx_cache=idx, ws=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ic.run_stack(pattern, layers, cfg.k, chunk=chunk, outs=outs, idx_cache=idx, ws=ws)
    g = torch.Generator(device="cuda").manual_seed(11)
    for rep in range(1, 4):
        for lay in layers:                                     # new small-integer inputs in place
            for name in ("q", "kv", "q_I", "k_I"):
                if name in lay:
                    lay[name].copy_(torch.randint(-3, 4, lay[name].shape, generator=g, device="cuda").to(lay[name].dtype))
            if "w" in lay:
                lay["w"].copy_(torch.randint(0, 4, lay["w"].shape, generator=g, device="cuda").to(lay["w"].dtype))
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        got_idx = idx.clone()
        ref_outs, ref_idx, _ = ic.run_stack(pattern, layers, cfg.k, chunk=chunk)
        torch.cuda.synchronize()
        assert torch.equal(got_idx, ref_idx), f"replay {rep}: idx differs"
        for l in range(len(pattern)):
            assert torch.equal(got[l], ref_outs[l]), f"replay {rep}: layer {l} differs"


def test_prefill_stacks_on_two_caller_streams():
    """Two run_stack calls in flight at once on two caller streams (they share the side
    stream) give the same results as the same calls made one after the other."""
    cfg = synth.WORKLOADS["tiny"]
    a = synth.prefill_stack(cfg, device="cuda", pattern="FSSS")
    b = [{k: v.flip(1).contiguous() for k, v in lay.items()}                # other inputs, F layers at 0 and 2
         for lay in synth.prefill_stack(cfg, device="cuda", pattern="FSFS")]
    ref_a = ic.run_stack("FSSS", a, cfg.k, chunk=128)
    ref_b = ic.run_stack("FSFS", b, cfg.k, chunk=64)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        got_a = ic.run_stack("FSSS", a, cfg.k, chunk=128, stream=s1)
    with torch.cuda.stream(s2):
        got_b = ic.run_stack("FSFS", b, cfg.k, chunk=64, stream=s2)
    torch.cuda.synchronize()
    for ref, got in ((ref_a, got_a), (ref_b, got_b)):
        assert torch.equal(ref[1], got[1])
        assert all(torch.equal(x, y) for x, y in zip(ref[0], got[0]))


def test_prefill_stack_one_tile_workspace_matches_two():
    """run_stack with the minimum workspace (one score tile: every top-k on the caller's
    stream) gives bitwise the results of the two-tile pipeline (top-k on the side stream)."""
    cfg = synth.WORKLOADS["tiny"]
    pattern, chunk = "FSFS", 128
    layers = synth.prefill_stack(cfg, device="cuda", pattern=pattern)
    shape = ic._stack_shape(pattern, layers, cfg.k, chunk, 0)
    two = ic.workspace_size(shape, ic.IC_OP_RUN_STACK)
    one = ic.workspace_size(shape, ic.IC_OP_INDEXER_TOPK)
    assert two >= 2 * one
    res = []
    for nbytes in (one, two):
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        res.append(ic.run_stack(pattern, layers, cfg.k, chunk=chunk, ws=ws))
    torch.cuda.synchronize()
    assert torch.equal(res[0][1], res[1][1])
    assert all(torch.equal(a, b) for a, b in zip(res[0][0], res[1][0]))


def _refill(lays, g):
    """New small-integer inputs in place (the captured graph keeps the same buffers)."""
    for lay in lays:
        for name in ("q", "kv", "q_I", "k_I"):
            if name in lay:
                lay[name].copy_(torch.randint(-3, 4, lay[name].shape, generator=g, device="cuda").to(lay[name].dtype))
        if "w" in lay:
            lay["w"].copy_(torch.randint(0, 4, lay["w"].shape, generator=g, device="cuda").to(lay["w"].dtype))


def test_varlen_stack_graph_replays_match_eager():
    """run_stack_varlen (its sequence tables travel by value in the kernel arguments: one
    group of two sequences, an empty sequence, one sequence longer than a chunk) captured in
    a graph: every replay with new inputs equals the eager call, bitwise."""
    q_len, pos0 = [100, 0, 37, 300], [0, 10, 200, 50]
    B, T, Lk = len(q_len), sum(q_len), 400
    H_I, d_I, k, H, d, chunk = 4, 32, 64, 4, 64, 128
    pattern = "FSFS"
    layers = []
    for c in pattern:
        lay = {"q": torch.zeros((T, H, d), dtype=torch.bfloat16, device="cuda"),
               "kv": torch.zeros((B, Lk, 2, d), dtype=torch.bfloat16, device="cuda")}
        if c == "F":
            lay.update(q_I=torch.zeros((T, H_I, d_I), dtype=torch.bfloat16, device="cuda"),
                       w=torch.zeros((T, H_I), dtype=torch.float32, device="cuda"),
                       k_I=torch.zeros((B, Lk, d_I), dtype=torch.bfloat16, device="cuda"))
        layers.append(lay)
    g = torch.Generator(device="cuda").manual_seed(21)
    _refill(layers, g)
    outs = [torch.empty_like(l["q"]) for l in layers]
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    run = lambda: ic.run_stack_varlen(pattern, layers, k, q_len, pos0, chunk=chunk, outs=outs, idx_cache=idx)
    run()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(1, 4):
        _refill(layers, g)
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        got_idx = idx.clone()
        ref_outs, ref_idx, _ = ic.run_stack_varlen(pattern, layers, k, q_len, pos0, chunk=chunk)
        torch.cuda.synchronize()
        assert torch.equal(got_idx, ref_idx), f"replay {rep}: idx differs"
        for l in range(len(pattern)):
            assert torch.equal(got[l], ref_outs[l]), f"replay {rep}: layer {l} differs"


def test_dynamic_stack_graph_replays_follow_their_inputs():
    """run_stack_dynamic captured in a graph.  The refresh decision stays on the device, so a
    replay must take each layer's decision from its own inputs: replays whose first S layer
    repeats the F layer's indexer inputs keep the cache there (its probe finds its own top-k),
    the others refresh.  Every replay equals the eager call: outputs, cache, decisions and
    recalls, bitwise."""
    cfg = synth.WORKLOADS["tiny"]
    pattern, chunk, stride, tau = "FSSS", 128, 16, 0.5
    layers = synth.prefill_stack(cfg, device="cuda", pattern="FFFF")   # every layer can probe
    outs = [torch.empty_like(l["q"]) for l in layers]
    idx = torch.empty((1, cfg.L, cfg.k), dtype=torch.int32, device="cuda")
    run = lambda: ic.run_stack_dynamic(pattern, layers, cfg.k, stride, tau, chunk=chunk, outs=outs, idx_cache=idx)
    run()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _, _, _, refreshed, recall = run()
    g = torch.Generator(device="cuda").manual_seed(23)
    seen = set()
    for rep in range(1, 5):
        _refill(layers, g)
        if rep % 2:
            for name in ("q_I", "w", "k_I"):
                layers[1][name].copy_(layers[0][name])
        graph.replay()
        torch.cuda.synchronize()
        got = ([o.clone() for o in outs], idx.clone(), refreshed.clone(), recall.clone())
        ref_outs, ref_idx, _, ref_ref, ref_rec = ic.run_stack_dynamic(pattern, layers, cfg.k, stride, tau, chunk=chunk)
        torch.cuda.synchronize()
        assert torch.equal(got[1], ref_idx), f"replay {rep}: idx differs"
        assert torch.equal(got[2], ref_ref), f"replay {rep}: decisions differ"
        assert torch.equal(torch.nan_to_num(got[3], nan=-1.0), torch.nan_to_num(ref_rec, nan=-1.0))
        for l in range(len(pattern)):
            assert torch.equal(got[0][l], ref_outs[l]), f"replay {rep}: layer {l} differs"
        seen.add(int(got[2][1, 0]))
        assert int(got[2][1, 0]) == (0 if rep % 2 else 1), f"replay {rep}: layer 1 decision {int(got[2][1, 0])}"
    assert seen == {0, 1}


def test_prefill_stacks_from_two_host_threads():
    """Two host threads, each on its own stream, calling run_stack three times on their own
    inputs at once (the library's error strings and counters are per thread; its second
    stream and scratch lookups are created under a lock): every result equals the same call
    made alone."""
    import threading
    cfg = synth.WORKLOADS["tiny"]
    inputs = [synth.prefill_stack(cfg, device="cuda", pattern="FSSS"),
              [{k: v.flip(1).contiguous() for k, v in lay.items()}
               for lay in synth.prefill_stack(cfg, device="cuda", pattern="FSFS")]]
    patterns, chunks = ("FSSS", "FSFS"), (128, 96)
    refs = [ic.run_stack(p, lays, cfg.k, chunk=c) for p, lays, c in zip(patterns, inputs, chunks)]
    torch.cuda.synchronize()
    results, errors = [[], []], []

    def work(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(3):
                    outs, idx, stats = ic.run_stack(patterns[i], inputs[i], cfg.k, chunk=chunks[i], stream=s)
                    results[i].append((outs, idx, stats))
            s.synchronize()
        except Exception as e:                                    # reported below, in the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        assert len(results[i]) == 3
        for outs, idx, stats in results[i]:
            assert stats == refs[i][2]
            assert torch.equal(idx, refs[i][1])
            assert all(torch.equal(a, b) for a, b in zip(outs, refs[i][0]))
