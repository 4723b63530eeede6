#!/usr/bin/env python3
"""Benchmark of the IndexCache / DSA hot path on one MI355X.

Workload (one timed step = one prefill pass through the whole stack):
  stack32k  B=1, L=32768 tokens, 16 layers 'FSSS'x4 (one indexer kept per four
            layers), lightning indexer H_I=64, d_I=128 in fp8 e4m3 with fp32
            accumulation, top-k 2048, sparse attention H=16 heads on one KV
            head, d=128, bf16.
After the timed prefill steps the same run measures, outside the timed loop:
  decode    decode64k: B=32 sequences with 65536 cached tokens, 24 layers
            'FSSS'x6, 64 decode steps (one new token per sequence per step);
  kernels   each kernel of the path timed alone with HIP events on the stream
            it runs on, priced against its roofline (MFMA for the indexer, HBM
            for top-k and gather attention), plus the fp8 MFMA rate this GPU
            sustains on constant and on random operands (libicprobe.so);
  all-F     the same stack with every layer running its indexer (the
            comparison the pages' prefill speedups are quoted against);
  oracle    the CPU oracle on a bounded sample of tokens (cpu_baseline).

Prints ONE JSON line.  Inputs are seeded synthetic tensors generated on the
GPU, resident in HBM before timing starts.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"fp8": 5000.0, "bf16": 2500.0}
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "dsa_lightning_indexer_scores_amd", "csrc")
KERNEL_SOURCES = {"indexer": "indexer.hip", "topk": "topk.hip", "attention": "attn.hip", "distill": "distill.hip"}
# launch grid of the whole-layer stack32k indexer in the kernel trace (8-query blocks x 2 key segments)
INDEXER_WHOLE_GRID = "4096x2"


def kernel_source_hash(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for name in (KERNEL_SOURCES[kernel], "common.h"):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary
    (scaled by the copy-kernel calibration), or None if absent or if the kernel source
    has changed since the counters were taken."""
    path = os.path.join(PROFILES, f"{kernel}_stack32k_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                vals[key.strip()] = val.strip()
    if vals.get("source_sha256") != kernel_source_hash(kernel):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def profile_value(fname: str, kernel: str, key: str):
    """A figure from a committed profile summary, or None if absent or taken on another
    source of the kernel."""
    path = os.path.join(PROFILES, fname)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != kernel_source_hash(kernel):
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def profile_grid_ms(fname: str, kernel: str, name_prefix: str, grid: str):
    """Average duration (ms) of one kernel's launches of one grid in a committed kernel-trace
    summary, or None if absent or taken on another source of the kernel."""
    path = os.path.join(PROFILES, fname)
    if not os.path.exists(path):
        return None
    ok, ms = False, None
    with open(path) as f:
        for line in f:
            if line.startswith(f"source_sha256.{kernel}:"):
                ok = line.split(":", 1)[1].strip() == kernel_source_hash(kernel)
            parts = line.split()
            if line.startswith(name_prefix) and grid in parts:
                i = parts.index(grid)
                ms = float(parts[i + 2]) / 1e3            # grid, calls, avg_us
    return ms if ok else None


def profile_kernel_us(fname: str, kernel: str, name: str):
    """Mean duration (us) of every launch of one kernel (exact name) in a committed
    kernel-trace summary, or None if absent or taken on another source of the kernel."""
    path = os.path.join(PROFILES, fname)
    if not os.path.exists(path):
        return None
    ok, us = False, None
    with open(path) as f:
        for line in f:
            if line.startswith(f"source_sha256.{kernel}:"):
                ok = line.split(":", 1)[1].strip() == kernel_source_hash(kernel)
            if us is None and line.startswith(name + " "):
                parts = line[len(name):].split()       # calls, avg_us, ...
                us = float(parts[1])
    return us if ok else None


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--decode-steps", type=int, default=64)
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-kernels", action="store_true")
    p.add_argument("--no-allf", action="store_true")
    p.add_argument("--no-long", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-share", action="store_true")
    p.add_argument("--no-varlen", action="store_true")
    p.add_argument("--cpu-tokens", type=int, default=640)
    p.add_argument("--only", choices=["indexer", "topk", "attention", "distill", "decode", "copy", "mfma"], default=None,
                   help="run just one kernel of the path a few times (for profiler counter runs)")
    p.add_argument("--reps", type=int, default=3)
    return p.parse_args()


def only_kernel(which: str, reps: int):
    """Launch one kernel of the path `reps` times on the stack32k inputs (or a 1 GiB copy),
    so that a profiler's counters cover exactly that kernel.  Prints one JSON line."""
    import torch
    import dsa_lightning_indexer_scores_amd as ic
    from dsa_lightning_indexer_scores_amd import synth
    cfg = synth.WORKLOADS["stack32k"]
    L, k = cfg.L, cfg.k
    info = {"only": which, "reps": reps}
    if which == "copy":
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(reps):
            dst.copy_(src)
        info.update(bytes_read=n, bytes_written=n)
    elif which == "decode":
        info.update(bench_decode(4, warm=1)[0])
    elif which == "mfma":
        info.update(mfma_ceiling() or {})
    else:
        layers = synth.prefill_stack(cfg, device="cuda", pattern="FSSS" if which == "distill" else "FS")
        f = layers[0]
        scores = torch.empty((1, L, L), dtype=torch.float32, device="cuda")
        ic.indexer_scores(f["q_I"], f["w"], f["k_I"], scores=scores, row_stride=L)
        idx = torch.empty((L, k), dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        if which == "indexer":
            for _ in range(reps):
                ic.indexer_scores(f["q_I"], f["w"], f["k_I"], scores=scores, row_stride=L)
        ic.topk_rows(scores[0], 1, k, idx=idx)
        if which == "topk":
            for _ in range(reps):
                ic.topk_rows(scores[0], 1, k, idx=idx)
        if which == "attention":
            del scores
            o = torch.empty_like(layers[1]["q"])
            for _ in range(reps):
                ic.sparse_attn(layers[1]["q"], layers[1]["kv"], idx.view(1, L, k), out=o)
        if which == "distill":
            del scores
            for _ in range(reps):
                ic.distill_kl(f["q_I"], f["w"], f["k_I"], idx.view(1, L, k), [l["q"] for l in layers],
                              [l["kv"] for l in layers], chunk=cfg.chunk)
    torch.cuda.synchronize()
    print(json.dumps(info), flush=True)


def timed_events(fn, reps: int):
    """Average ms of fn() over reps, bracketed by HIP events on the current stream."""
    import torch
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        fn()
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def kernel_rooflines(cfg, layers, ws):
    """Time each kernel of the prefill path alone; return per-kernel roofline entries."""
    import torch
    import dsa_lightning_indexer_scores_amd as ic
    L, k = cfg.L, cfg.k
    f = layers[0]
    pairs = L * (L + 1) // 2
    out = {}
    # a1: indexer scores over the full causal triangle (one launch, all 32768 queries)
    scores = torch.empty((1, L, L), dtype=torch.float32, device="cuda")
    ic.indexer_scores(f["q_I"], f["w"], f["k_I"], scores=scores, row_stride=L)
    ms = timed_events(lambda: ic.indexer_scores(f["q_I"], f["w"], f["k_I"], scores=scores, row_stride=L), 3)
    flops = 2.0 * cfg.H_I * cfg.d_I * pairs
    tf = flops / (ms * 1e-3) / 1e12
    out["indexer"] = {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_TFLOPS[cfg.idx_dtype],
                      "unit": "TFLOP/s", "frac": round(tf / PEAK_TFLOPS[cfg.idx_dtype], 4), "ms": round(ms, 4),
                      "work": f"{flops:.4g} flop = 2*H_I*d_I per causal pair x {pairs} pairs"}
    # the same layer in the 4096-query tiles the stack launches (8 launches)
    ch = cfg.chunk
    tile = torch.empty(ch * L, dtype=torch.float32, device="cuda")

    def chunked():
        for c0 in range(0, L, ch):
            n = min(ch, L - c0)
            rs = (c0 + n + 3) // 4 * 4
            ic.indexer_scores(f["q_I"][:, c0:c0 + n], f["w"][:, c0:c0 + n], f["k_I"], pos0=c0,
                              scores=tile[:n * rs].view(1, n, rs), row_stride=rs)
    chunked()
    ms_c = timed_events(chunked, 3)
    out["indexer"]["chunked_ms"] = round(ms_c, 4)
    out["indexer"]["chunked_frac"] = round(flops / (ms_c * 1e-3) / 1e12 / PEAK_TFLOPS[cfg.idx_dtype], 4)
    del tile
    # a2: top-k over those rows (one launch, 32768 rows)
    sc2 = scores[0]
    idx = torch.empty((L, k), dtype=torch.int32, device="cuda")
    ic.topk_rows(sc2, 1, k, idx=idx)
    ms = timed_events(lambda: ic.topk_rows(sc2, 1, k, idx=idx), 3)
    by = 4.0 * pairs + 4.0 * k * L
    gbs = by / (ms * 1e-3) / 1e9
    out["topk"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                   "frac": round(gbs / PEAK_HBM_GBS, 4), "ms": round(ms, 4),
                   "work": f"{by:.4g} B = 4 B per visible score + 4k B idx per query"}
    # the same rows in the 4096-row launches the stack makes (each picks its shape by its rows' length)

    def topk_chunked():
        for c0 in range(0, L, ch):
            ic.topk_rows(sc2[c0:c0 + ch], c0 + 1, k, idx=idx[c0:c0 + ch])
    topk_chunked()
    ms_tc = timed_events(topk_chunked, 3)
    out["topk"]["chunked_ms"] = round(ms_tc, 4)
    out["topk"]["chunked_frac"] = round(by / (ms_tc * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    del scores
    # a4: gather attention of one layer with those indices
    idx3 = idx.view(1, L, k)
    o = torch.empty_like(layers[1]["q"])
    ic.sparse_attn(layers[1]["q"], layers[1]["kv"], idx3, out=o)
    ms = timed_events(lambda: ic.sparse_attn(layers[1]["q"], layers[1]["kv"], idx3, out=o), 5)
    rows = int((idx3 >= 0).sum().item())
    by = 512.0 * rows + L * (cfg.H * cfg.d * 2 * 2 + 4 * k)
    gbs = by / (ms * 1e-3) / 1e9
    # The gathered rows come mostly from L2 / MALL (the layer's KV is 16.8 MB), so the
    # algorithmic rate is a cache gather rate, not an HBM one, and no HBM `frac` is given;
    # the HBM rate is the counter traffic over the same time (added in main).
    out["attention"] = {"bound": "gather from L2/MALL (address unit)", "algorithmic_gbs": round(gbs, 1),
                        "unit": "GB/s", "ms": round(ms, 4),
                        "work": f"{by:.4g} B = 512 B per selected [K|V] row x {rows} rows + q, out, idx"}
    g_ms = gather_ceiling_ms(layers[1]["kv"], idx3)
    if g_ms:
        # the same rows read by a kernel that does nothing else (libicprobe.so): the
        # attention's address stream without its math
        out["attention"]["gather_only_ms"] = round(g_ms, 4)
        out["attention"]["frac_of_gather_only"] = round(g_ms / ms, 4)
    # NEXT-3: distillation loss forward of the first F layer serving itself and its three S layers
    # (the call recomputes the indexer scores in the stack's tiles; the loss kernel's own time is
    # the call minus those indexer launches, timed above as chunked_ms)
    if len(layers) >= 4:
        served = layers[:4]
        kl = torch.empty((1, L), dtype=torch.float32, device="cuda")
        mean = torch.empty(1, dtype=torch.float32, device="cuda")
        run = lambda: ic.distill_kl(f["q_I"], f["w"], f["k_I"], idx3, [l["q"] for l in served],
                                    [l["kv"] for l in served], chunk=cfg.chunk, kl=kl, mean=mean)
        run()
        ms_call = timed_events(run, 3)
        ms_k = max(ms_call - out["indexer"]["chunked_ms"], 1e-6)
        by = 256.0 * rows * len(served) + L * (len(served) * cfg.H * cfg.d * 2 + 4 * k + 4 * k + 4)
        gbs = by / (ms_k * 1e-3) / 1e9
        # like the attention, the served layers' K rows (16.8 MB each) come mostly from L2 / MALL:
        # the algorithmic rate is a cache gather rate, and the HBM rate is the counter traffic
        out["distill"] = {"bound": "gather from L2/MALL (address unit)", "algorithmic_gbs": round(gbs, 1),
                          "unit": "GB/s", "ms": round(ms_k, 4), "call_ms": round(ms_call, 4),
                          "served_layers": len(served), "loss_mean_nats": round(float(mean.item()), 4),
                          "work": f"{by:.4g} B = 256 B K per (selected row, served layer) x {rows} rows x "
                                  f"{len(served)} + q, idx, scores, kl (read twice: two sweeps)",
                          "method": "call minus the indexer's tiled launches",
                          "launches": (L + cfg.chunk - 1) // cfg.chunk}
    return out


def bench_long():
    """long128k (one 131072-token sequence, 8 layers 'FSSSSSSS'): ms per step of the
    pattern and of the all-F stack on the same seeded layers, the closest in-build
    analogue of the pages' long-context speedups."""
    import torch
    import dsa_lightning_indexer_scores_amd as ic
    from dsa_lightning_indexer_scores_amd import synth
    cfg = synth.WORKLOADS["long128k"]
    layers = synth.prefill_stack(cfg, device="cuda", pattern="F" * len(cfg.pattern))
    outs = [torch.empty_like(l["q"]) for l in layers]
    idx = torch.empty((cfg.B, cfg.L, cfg.k), dtype=torch.int32, device="cuda")
    shape = ic._stack_shape(cfg.pattern, layers, cfg.k, cfg.chunk, 0)
    ws = torch.empty(ic.workspace_size(shape, ic.IC_OP_RUN_STACK), dtype=torch.uint8, device="cuda")
    out = {"workload": f"long128k: B=1, L={cfg.L}, {len(cfg.pattern)} layers '{cfg.pattern}', H_I=64, d_I=128 fp8, "
                       f"k={cfg.k}, H=16, d=128 bf16"}
    ms = {}
    for name, pat, n in (("pattern", cfg.pattern, 3), ("all_f", "F" * len(cfg.pattern), 2)):
        ic.run_stack(pat, layers, cfg.k, chunk=cfg.chunk, outs=outs, idx_cache=idx, ws=ws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            ic.run_stack(pat, layers, cfg.k, chunk=cfg.chunk, outs=outs, idx_cache=idx, ws=ws)
        torch.cuda.synchronize()
        ms[name] = (time.perf_counter() - t0) * 1e3 / n
    out["ms_per_step"] = round(ms["pattern"], 3)
    out["tokens_per_s"] = round(cfg.B * cfg.L / (ms["pattern"] * 1e-3), 1)
    out["all_f_ms_per_step"] = round(ms["all_f"], 3)
    out["speedup_of_pattern"] = round(ms["all_f"] / ms["pattern"], 3)
    del layers, outs, idx, ws
    torch.cuda.empty_cache()
    return out


def bench_varlen(n_seq: int = 64, q_new: int = 512, Lk: int = 8192, seed: int = 77):
    """Ragged batched prefill, the serving case: n_seq sequences each bring q_new queries that
    continue a cached prefix of 0 .. Lk - q_new tokens, through the 16-layer FSSS stack with the
    stack32k layer shapes.  One ic_run_stack_varlen call (consecutive sequences share
    launches) against one ic_run_stack per sequence on the same tensors."""
    import torch
    import dsa_lightning_indexer_scores_amd as ic
    from dsa_lightning_indexer_scores_amd import synth
    cfg = synth.WORKLOADS["stack32k"]
    layers, q_len, pos0 = synth.ragged_stack(cfg, n_seq, q_new, Lk, seed, device="cuda")
    T = n_seq * q_new
    outs = [torch.empty_like(l["q"]) for l in layers]
    idx = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    grouped = lambda: ic.run_stack_varlen(cfg.pattern, layers, cfg.k, q_len, pos0, outs=outs, idx_cache=idx)
    per_seq_layers = []
    for b in range(n_seq):
        q0 = b * q_new
        one = []
        for lay in layers:
            o = {"q": lay["q"][q0:q0 + q_new].unsqueeze(0), "kv": lay["kv"][b:b + 1]}
            if "q_I" in lay:
                o.update(q_I=lay["q_I"][q0:q0 + q_new].unsqueeze(0), w=lay["w"][q0:q0 + q_new].unsqueeze(0),
                         k_I=lay["k_I"][b:b + 1])
            one.append(o)
        per_seq_layers.append(one)
    shape1 = ic._stack_shape(cfg.pattern, per_seq_layers[0], cfg.k, 0, 0)
    ws1 = torch.empty(ic.workspace_size(ic.make_shape(1, q_new, Lk, cfg.k, cfg.H, cfg.d, cfg.H_I, cfg.d_I,
                                                      ic.IC_FP8_E4M3, pos0=Lk - q_new), ic.IC_OP_RUN_STACK),
                      dtype=torch.uint8, device="cuda")
    del shape1
    outs1 = [[o[b * q_new:(b + 1) * q_new].unsqueeze(0) for o in outs] for b in range(n_seq)]

    def per_sequence():
        for b in range(n_seq):
            ic.run_stack(cfg.pattern, per_seq_layers[b], cfg.k, pos0=pos0[b], outs=outs1[b],
                         idx_cache=idx[b * q_new:(b + 1) * q_new].unsqueeze(0), ws=ws1)
    grouped()
    per_sequence()
    t_g = timed_events(grouped, 3)
    t_p = timed_events(per_sequence, 3)
    del layers, outs, idx, per_seq_layers, outs1, ws1
    torch.cuda.empty_cache()
    return {"workload": f"ragged prefill: {n_seq} sequences x {q_new} new tokens continuing prefixes of 0..{Lk - q_new}, "
                        f"16 layers 'FSSS'x4, stack32k layer shapes",
            "grouped_ms": round(t_g, 3), "tokens_per_s": round(T / (t_g * 1e-3), 1),
            "per_sequence_ms": round(t_p, 3), "speedup_of_grouping": round(t_p / t_g, 3)}


def gather_ceiling_ms(kv, idx3):
    """Time of a pure gather of the rows idx3 [1, L, k] names from kv [1, L, 2, d] (libicprobe.so)."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "dsa_lightning_indexer_scores_amd", "libicprobe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.icp_gather_rows.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    nq, k = idx3.shape[1], idx3.shape[2]
    Lk, row_bytes = kv.shape[1], kv.shape[2] * kv.shape[3] * 2
    out = torch.empty(nq * 64, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()

    def launch():
        r = lib.icp_gather_rows(ctypes.c_void_p(kv.data_ptr()), ctypes.c_void_p(idx3.data_ptr()), nq, k, Lk, row_bytes,
                                ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(st.cuda_stream))
        if r != 0:
            raise RuntimeError(f"icp_gather_rows failed: hipError {r}")
    launch()
    return timed_events(launch, 5)


def mfma_ceiling():
    """Sustained fp8 MFMA rate of this GPU, as fractions of the 5.0 PFLOP/s peak: a
    stream of independent 16x16x128 fp8 MFMAs (libicprobe.so) over constant operands,
    over random operands that change every iteration as the indexer's keys do, with the
    indexer's own operand pattern, and with that pattern plus the indexer's vector
    epilogue (its whole instruction mix without memory traffic)."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "dsa_lightning_indexer_scores_amd", "libicprobe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.icp_mfma_stream.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    blocks, iters = 8192, 2048
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream()
    res = {}
    for name, rnd, per_iter in (("constant_operands", 0, 8), ("random_operands", 1, 8),
                                ("indexer_operands", 2, 9), ("indexer_compute", 3, 9)):
        def launch():
            r = lib.icp_mfma_stream(rnd, blocks, iters, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(st.cuda_stream))
            if r != 0:
                raise RuntimeError(f"icp_mfma_stream failed: hipError {r}")
        launch()
        ms = timed_events(launch, 3)
        flops = per_iter * 65536.0 * iters * blocks * 4
        res[name] = round(flops / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["fp8"], 4)
    return res


def stream_read_gbs(nbytes: int = 1 << 30) -> float:
    """HBM read bandwidth of a plain streaming kernel over a 1 GiB buffer (libicprobe.so)."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "dsa_lightning_indexer_scores_amd", "libicprobe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.icp_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    blocks = 4096
    out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()

    def launch():
        r = lib.icp_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, blocks, ctypes.c_void_p(out.data_ptr()),
                                ctypes.c_void_p(st.cuda_stream))
        if r != 0:
            raise RuntimeError(f"icp_stream_read failed: hipError {r}")
    launch()
    ms = timed_events(launch, 5)
    return round(nbytes / (ms * 1e-3) / 1e9, 1)


def cpu_baseline(cfg, layers, n_tokens: int, seed: int = 7):
    """Time the oracle on n_tokens query positions drawn uniformly from the sequence,
    each taken through every layer of the stack (F: indexer + top-k + attention; S: attention)."""
    import numpy as np
    import oracle as O
    from dsa_lightning_indexer_scores_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    rng = np.random.default_rng(seed)
    pos = np.sort(rng.choice(cfg.L, size=n_tokens, replace=False))
    pos_t = __import__("torch").from_numpy(pos).cuda()
    ref = []
    for c, lay in zip(cfg.pattern, layers):
        r = {"q": O.decode_bf16(synth.bits_u16(lay["q"][0].index_select(0, pos_t))),
             "kv": O.decode_bf16(synth.bits_u16(lay["kv"][0]))}
        if c in "F1":
            dq = O.decode_e4m3 if cfg.idx_dtype == "fp8" else O.decode_bf16
            raw = synth.bits_u8 if cfg.idx_dtype == "fp8" else synth.bits_u16
            r["q_I"] = dq(raw(lay["q_I"][0].index_select(0, pos_t)))
            r["w"] = lay["w"][0].index_select(0, pos_t).double().cpu().numpy()
            r["k_I"] = dq(raw(lay["k_I"][0]))
        ref.append(r)
    scale = 1.0 / np.sqrt(cfg.d)
    t0 = time.perf_counter()
    for i, p in enumerate(pos):
        cache = None
        for c, r in zip(cfg.pattern, ref):
            if c in "F1":
                cache = O.topk_row(O.to_decision_precision(O.indexer_scores_row(r["q_I"][i], r["w"][i], r["k_I"], int(p))),
                                   cfg.k)
            O.sparse_attn_row(r["q"][i], r["kv"], cache, scale)
    dt = time.perf_counter() - t0
    return {"value": round(n_tokens / dt, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_tokens} query positions drawn uniformly from the 32768-token prefill, each through "
                      f"all {len(cfg.pattern)} layers ('FSSS'x4) of the same seeded inputs; fp64 numpy oracle, "
                      f"{dt:.1f} s"}


def bench_decode(n_steps: int, warm: int = 2, pattern: str = None, caches=None, kernels: bool = True):
    """decode64k: the steps replay one captured HIP graph of ic_decode_step.

    Each step's new queries (q for every layer, q_I and w for F layers) and the
    sequence lengths live in one static input buffer; per step a single
    device-to-device copy loads that step's seeded inputs into it, then the
    graph replays.  Both the copy and the replay are inside the timed loop.
    pattern overrides the workload's ('F' * 24 is the all-F stack on the same
    caches, with indexer keys added for every layer); caches are reused if given.
    Returns (result dict, caches).
    """
    import torch
    import dsa_lightning_indexer_scores_amd as ic
    from dsa_lightning_indexer_scores_amd import synth
    cfg = synth.WORKLOADS["decode64k"]
    pattern = cfg.pattern if pattern is None else pattern
    total = warm + n_steps
    steps_cap = max(total, cfg.decode_steps)
    if caches is None:
        caches = synth.decode_caches(cfg, device="cuda", steps=steps_cap, pattern=pattern)
    cap_steps = caches[0]["kv"].shape[1] - cfg.L               # rows the caches hold past the context
    for l, c in enumerate(pattern):
        if c in "F1" and "k_I" not in caches[l]:
            caches[l]["k_I"] = synth.decode_k_I(cfg, l, device="cuda", steps=cap_steps)
    # static input buffer layout: per layer q (+ q_I, w), then seq_len
    first = synth.decode_queries(cfg, 0, device="cuda", pattern=pattern)
    parts = []
    for lay in first:
        for name in ("q", "q_I", "w"):
            if name in lay:
                parts.append((lay[name].dtype, tuple(lay[name].shape), lay[name].numel() * lay[name].element_size()))
    parts.append((torch.int32, (cfg.B,), 4 * cfg.B))
    nbytes = sum(-(-p[2] // 256) * 256 for p in parts)
    static = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    pregen = torch.empty((total, nbytes), dtype=torch.uint8, device="cuda")

    def views(buf):
        out, off = [], 0
        for dt, shape, nb in parts:
            out.append(buf[off:off + nb].view(dt).view(shape))
            off += -(-nb // 256) * 256
        return out

    for s_ in range(total):
        qs = first if s_ == 0 else synth.decode_queries(cfg, s_, device="cuda", pattern=pattern)
        flat = [lay[name] for lay in qs for name in ("q", "q_I", "w") if name in lay]
        flat.append(torch.full((cfg.B,), cfg.L + s_ + 1, dtype=torch.int32, device="cuda"))
        for dst, src in zip(views(pregen[s_]), flat):
            dst.copy_(src)
    sv = views(static)
    layers, i = [], 0
    for l, c in enumerate(pattern):
        lay = {"kv": caches[l]["kv"]}
        lay["q"] = sv[i]; i += 1
        if c in "F1":
            lay["k_I"] = caches[l]["k_I"]
            lay["q_I"] = sv[i]; lay["w"] = sv[i + 1]; i += 2
        layers.append(lay)
    seq_len = sv[i]
    outs = [torch.empty_like(l["q"]) for l in layers]
    idx_cache = torch.empty((cfg.B, 1, cfg.k), dtype=torch.int32, device="cuda")
    shape = ic._stack_shape(pattern, layers, cfg.k, 0, 0)
    ws = torch.empty(ic.workspace_size(shape, ic.IC_OP_DECODE_STEP), dtype=torch.uint8, device="cuda")
    static.copy_(pregen[0])
    ic.decode_step(pattern, layers, seq_len, cfg.k, outs=outs, idx_cache=idx_cache, ws=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ic.decode_step(pattern, layers, seq_len, cfg.k, outs=outs, idx_cache=idx_cache, ws=ws)
    for s_ in range(warm):
        static.copy_(pregen[s_])
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(warm, total):
        static.copy_(pregen[s_])
        g.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    res = {"tokens_per_s": round(cfg.B * n_steps / dt, 1), "ms_per_step": round(dt * 1e3 / n_steps, 4),
           "steps": n_steps,
           "workload": f"decode64k: B=32, 65536 cached tokens, 24 layers '{pattern[:4]}'x6, k=2048, fp8 indexer, "
                       f"H=16, d=128; one captured graph replayed per step"}
    if kernels:
        eager_t0 = time.perf_counter()
        for s_ in range(warm, min(total, warm + 8)):
            static.copy_(pregen[s_])
            ic.decode_step(pattern, layers, seq_len, cfg.k, outs=outs, idx_cache=idx_cache, ws=ws)
        torch.cuda.synchronize()
        res["eager_ms_per_step"] = round((time.perf_counter() - eager_t0) * 1e3 / min(n_steps, 8), 4)
        res["kernels"] = decode_kernel_rooflines(cfg, layers, seq_len, int(seq_len[0].item()))
    del pregen, static, g
    return res, caches


def decode_kernel_rooflines(cfg, layers, seq_len, n: int):
    """Decode is the honest HBM test (its caches do not fit on chip).  Each kernel of an F
    layer and an S layer runs alone through its own entry point on the step's caches and
    lengths (the launches ic_decode_step makes), timed with HIP events on the current stream:
    the indexer scores, the top-k of those scores (segment ranking, then the candidates), and
    the split-K attention with its merge."""
    import torch
    import dsa_lightning_indexer_scores_amd as ic
    B, k = cfg.B, cfg.k
    f, s_lay = layers[0], layers[1]
    cap = f["k_I"].shape[1]
    scores = torch.empty((B, (cap + 3) // 4 * 4), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    ws_t = torch.empty(max(ic.topk_rows_seq_ws(B, cap, k), 256), dtype=torch.uint8, device="cuda")
    run_idx = lambda: ic.decode_indexer_scores(f["q_I"], f["w"], f["k_I"], seq_len, scores=scores)
    run_topk = lambda: ic.topk_rows_seq(scores, seq_len, k, max_len=cap, idx=idx, ws=ws_t)
    run_idx()
    run_topk()
    idx3 = idx.view(B, 1, k)
    out = torch.empty_like(s_lay["q"])
    shape = ic.make_shape(B, 1, cap, k, cfg.H, cfg.d)
    ws_a = torch.empty(max(ic.workspace_size(shape, ic.IC_OP_DECODE_ATTN), 256), dtype=torch.uint8, device="cuda")
    run_attn = lambda: ic.decode_attn(s_lay["q"], s_lay["kv"], idx3, out=out, ws=ws_a)
    run_attn()
    t_idx = timed_events(run_idx, 20)
    t_topk = timed_events(run_topk, 20)
    t_attn = timed_events(run_attn, 20)
    rows = int((idx >= 0).sum().item())
    by_idx = B * n * cfg.d_I * 1.0 + B * n * 4.0               # k_I rows read + scores written
    by_topk = B * n * 4.0 + B * k * 4.0                       # scores read + idx written
    by_attn = rows * 512.0 + B * (cfg.H * cfg.d * 2 * 2 + 4 * k)   # selected rows + q, out, idx
    mk = lambda ms, by, what: {"bound": "hbm", "ms": round(ms, 5), "achieved": round(by / (ms * 1e-3) / 1e9, 1),
                               "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": round(by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "work": what}
    res = {"indexer": mk(t_idx, by_idx, f"{by_idx:.4g} B = 128 B k_I + 4 B score per (sequence, visible key)"),
           "topk": mk(t_topk, by_topk, f"{by_topk:.4g} B = 4 B per visible score + 4k B idx per sequence"),
           "attention": mk(t_attn, by_attn, f"{by_attn:.4g} B = 512 B per selected row + q, out, idx"),
           "method": "each kernel alone through its entry point, HIP events on the current stream"}
    # The same launches in the committed rocprofv3 trace (another box and run; its mean over the
    # trace's graph-replayed, eager and solo launches), read only while its kernel sources match.
    trace = "decode64k_kernel_trace.txt"
    parts = {"indexer": [("indexer", "indexer_decode_kernel<true, 128, 4>")],
             "topk": [("topk", "topk_kernel<1024, 16, true, false, 1>"), ("topk", "topk_kernel<1024, 16, true, false, 2>")],
             "attention": [("attention", "sparse_attn_split_kernel<128>"), ("attention", "attn_combine_kernel<128>")]}
    for name, launches in parts.items():
        us = [profile_kernel_us(trace, src, kname) for src, kname in launches]
        if all(u is not None for u in us):
            e = res[name]
            by = {"indexer": by_idx, "topk": by_topk, "attention": by_attn}[name]
            e["profile_us"] = round(sum(us), 2)
            e["profile_frac"] = round(by / (sum(us) * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
    return res


def indexer_share_curve(lengths=(8192, 32768, 131072)):
    """The indexer's share of a layer at several context lengths (the stack32k layer shapes:
    fp8 indexer H_I=64, d_I=128, k=2048, 16 heads, d=128): one F layer through ic_run_stack
    (indexer + top-k + attention, with the stack's overlap) against the same layer's attention
    alone.  An all-F stack spends (F - A) / F of its time on indexer and top-k; the FSSS
    pattern (F + 3 S) spends (F - A) / (F + 3 A)."""
    import dataclasses
    import torch
    import dsa_lightning_indexer_scores_amd as ic
    from dsa_lightning_indexer_scores_amd import synth
    base = synth.WORKLOADS["stack32k"]
    out = []
    for L in lengths:
        cfg = dataclasses.replace(base, L=L, pattern="F")
        lay = [synth.prefill_layer(cfg, 0, device="cuda")]
        outs = [torch.empty_like(lay[0]["q"])]
        idx = torch.empty((1, L, cfg.k), dtype=torch.int32, device="cuda")
        shape = ic._stack_shape("F", lay, cfg.k, cfg.chunk, 0)
        ws = torch.empty(ic.workspace_size(shape, ic.IC_OP_RUN_STACK), dtype=torch.uint8, device="cuda")
        run_f = lambda: ic.run_stack("F", lay, cfg.k, chunk=cfg.chunk, outs=outs, idx_cache=idx, ws=ws)
        run_a = lambda: ic.sparse_attn(lay[0]["q"], lay[0]["kv"], idx, out=outs[0])
        run_f()
        n = 3 if L <= 32768 else 2
        t_f = timed_events(run_f, n)
        t_a = timed_events(run_a, n)
        out.append({"L": L, "f_layer_ms": round(t_f, 3), "attention_ms": round(t_a, 3),
                    "indexer_share_all_f": round((t_f - t_a) / t_f, 4),
                    "indexer_share_fsss": round((t_f - t_a) / (t_f + 3 * t_a), 4)})
        del lay, outs, idx, ws
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(sequences and query blocks would shard across GPUs, but nothing here runs that); "
              "use --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.only:
        only_kernel(args.only, args.reps)
        return
    import torch
    import dsa_lightning_indexer_scores_amd as ic
    from dsa_lightning_indexer_scores_amd import synth

    cfg = synth.WORKLOADS["stack32k"]
    torch.cuda.set_device(0)
    log(f"generating {cfg.name} inputs on the GPU")
    layers = synth.prefill_stack(cfg, device="cuda")
    outs = [torch.empty_like(l["q"]) for l in layers]
    idx_cache = torch.empty((cfg.B, cfg.L, cfg.k), dtype=torch.int32, device="cuda")
    shape = ic._stack_shape(cfg.pattern, layers, cfg.k, 0, 0)
    ws = torch.empty(ic.workspace_size(shape, ic.IC_OP_RUN_STACK), dtype=torch.uint8, device="cuda")

    def step():
        return ic.run_stack(cfg.pattern, layers, cfg.k, outs=outs, idx_cache=idx_cache, ws=ws)

    for _ in range(args.warmup):
        _, _, stats = step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} prefill steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        _, _, stats = step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_step = dt * 1e3 / args.steps
    value = cfg.B * cfg.L / (dt / args.steps)
    log(f"prefill {ms_step:.2f} ms/step, {value:.0f} tokens/s, stats {stats}")

    result = {
        "metric": "stack prefill tokens/s @32K (FSSS) + decode tokens/s; indexer MFMA %",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8 indexer (fp32 accumulate) + bf16 attention", "data": "synthetic (seeded, generated on GPU)",
        "config": {"workload": "stack32k: B=1, L=32768, 16 layers 'FSSS'x4, H_I=64, d_I=128 fp8, k=2048, "
                               "H=16, d=128 bf16", "global_batch": cfg.B, "seq_len": cfg.L,
                   "parallelism": "single GPU"},
        "stack_stats": stats,
    }

    if not args.no_kernels:
        log("timing kernels alone")
        kr = kernel_rooflines(cfg, layers, ws)
        share = {"indexer": kr["indexer"]["chunked_ms"] * cfg.pattern.count("F"),
                 "topk": kr["topk"]["chunked_ms"] * cfg.pattern.count("F"),
                 "attention": kr["attention"]["ms"] * cfg.n_layers}
        dom = max(share, key=share.get)
        # The headline roofline is the indexer's: its MFMA bound binds (the metric's own
        # "indexer MFMA %"), and it is the O(L^2) term the pattern removes from S layers.
        # The gather attention takes more of the stack at 32K, but its layer's KV (16.8 MB)
        # is served from L2 / MALL, so no HBM roofline binds it: it is reported in `kernels`
        # by its counter-measured HBM traffic and against a pure gather of the same rows.
        ix = kr["indexer"]
        result["roofline"] = {"bound": "mfma", "achieved": ix["achieved"], "peak": ix["peak"], "unit": ix["unit"],
                              "frac": ix["frac"], "kernel": "indexer", "ms": ix["ms"],
                              "traffic": measured_traffic("indexer"), "work": ix["work"],
                              "largest_share_kernel": dom}
        # the same launch in the committed rocprofv3 trace (another box, another run): its
        # average duration and the fraction it gives, for the comparison with `ms`
        pms = profile_grid_ms("bench_stack32k_kernel_trace.txt", "indexer", "indexer_prefill_kernel<true",
                              INDEXER_WHOLE_GRID)
        if pms:
            result["roofline"]["profile_ms"] = round(pms, 4)
            result["roofline"]["profile_frac"] = round(ix["achieved"] * ix["ms"] / pms / ix["peak"], 4)
        for name in kr:
            t = measured_traffic(name)               # per dispatch; the distillation call makes one per tile
            kr[name]["traffic"] = None if t is None else t * kr[name].get("launches", 1)
        for name in ("attention", "distill"):
            at = kr.get(name)
            if at and at["traffic"] is not None:
                at["traffic_gbs"] = round(at["traffic"] / (at["ms"] * 1e6), 1)
                at["traffic_frac"] = round(at["traffic_gbs"] / PEAK_HBM_GBS, 4)
        at = kr["attention"]
        busy = profile_value("attention_stack32k_counters.txt", "attention", "address_unit_busy")
        if busy is not None:
            at["address_unit_busy"] = busy
        result["kernels"] = kr
        result["kernel_ms_in_stack"] = {k: round(v, 3) for k, v in share.items()}
        result["indexer_mfma_frac"] = kr["indexer"]["frac"]
        ceil = mfma_ceiling()
        if ceil:
            result["mfma_sustained_frac"] = ceil
            # the indexer's own operand pattern (fixed q_I slabs, fresh keys from LDS each
            # tile, the linear-term MFMA): 8 of its 9 MFMAs per tile are the algorithmic work
            result["indexer_frac_of_sustained"] = round(kr["indexer"]["frac"] / (ceil["indexer_operands"] * 8 / 9), 4)
            # the same stream with the indexer's vector epilogue (its whole arithmetic, no
            # memory traffic, key-block loads or barriers): the ceiling of its instruction mix
            if "indexer_compute" in ceil:
                result["indexer_frac_of_compute_mix"] = round(kr["indexer"]["frac"] / (ceil["indexer_compute"] * 8 / 9), 4)
        sgbs = stream_read_gbs()
        if sgbs:
            result["hbm_stream_read_gbs"] = sgbs
            kr["topk"]["frac_of_stream"] = round(kr["topk"]["achieved"] / sgbs, 4)

    if not args.no_allf:
        log("timing the all-F stack")
        allf = [dict(layers[(l // 4) * 4], q=layers[l]["q"], kv=layers[l]["kv"]) for l in range(cfg.n_layers)]
        pat = "F" * cfg.n_layers
        ic.run_stack(pat, allf, cfg.k, outs=outs, idx_cache=idx_cache, ws=ws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(2):
            ic.run_stack(pat, allf, cfg.k, outs=outs, idx_cache=idx_cache, ws=ws)
        torch.cuda.synchronize()
        allf_ms = (time.perf_counter() - t0) * 1e3 / 2
        result["all_f"] = {"ms_per_step": round(allf_ms, 3), "speedup_of_pattern": round(allf_ms / ms_step, 3)}

        # NEXT-4: the same stack where every S layer keeps its indexer and probes the cache on every
        # 64th query (drift-triggered refresh); tau = 0 never refreshes (the probes' cost alone),
        # tau > 1 always refreshes (every layer re-indexed, plus the probes)
        log("timing dynamic refresh")
        n_s = cfg.pattern.count("S")
        dyn = {"probe_stride": 64, "s_layers": n_s}
        for name, tau in (("never", 0.0), ("always", 1.01)):
            r = ic.run_stack_dynamic(cfg.pattern, allf, cfg.k, 64, tau, outs=outs, idx_cache=idx_cache)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(2):
                r = ic.run_stack_dynamic(cfg.pattern, allf, cfg.k, 64, tau, outs=outs, idx_cache=idx_cache)
            torch.cuda.synchronize()
            dyn[name + "_ms_per_step"] = round((time.perf_counter() - t0) * 1e3 / 2, 3)
            dyn[name + "_refreshed_layers"] = int((r[3] == 1).sum().item())
        dyn["probe_ms_per_s_layer"] = round((dyn["never_ms_per_step"] - ms_step) / max(n_s, 1), 4)
        result["dynamic_refresh"] = dyn

    if not args.no_long:
        log("timing long128k")
        result["long128k"] = bench_long()

    if not args.no_decode:
        log("timing decode64k")
        del outs
        result["decode"], caches = bench_decode(args.decode_steps)
        result["decode_tokens_per_s"] = result["decode"]["tokens_per_s"]
        sgbs = result.get("hbm_stream_read_gbs")
        if sgbs:
            for v in result["decode"]["kernels"].values():
                if isinstance(v, dict):
                    v["frac_of_stream"] = round(v["achieved"] / sgbs, 4)
        if not args.no_allf:
            # the same caches with indexer keys for every layer: the in-build analogue of the
            # pages' decode speedup (standard DSA runs the indexer at every layer)
            log("timing decode64k all-F")
            allf, _ = bench_decode(16, pattern="F" * len(synth.WORKLOADS["decode64k"].pattern), caches=caches,
                                   kernels=False)
            result["decode"]["all_f_ms_per_step"] = allf["ms_per_step"]
            result["decode"]["speedup_of_pattern"] = round(allf["ms_per_step"] / result["decode"]["ms_per_step"], 3)
        del caches
        torch.cuda.empty_cache()

    if not args.no_varlen:
        log("timing ragged prefill (64 sequences)")
        result["varlen"] = bench_varlen()

    if not args.no_share:
        log("timing the indexer share at 8K / 32K / 128K")
        result["indexer_share"] = indexer_share_curve()

    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(cfg, layers, args.cpu_tokens)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
