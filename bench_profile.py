#!/usr/bin/env python3
"""Reduce rocprofv3 CSV output to the short text summaries kept under profiles/.

  trace     a --kernel-trace CSV -> per-kernel calls / avg / min / max / total, and the
            same by launch grid for the kernels named with --grid
  counters  --pmc CSVs (one per pass) -> the mean per dispatch of every counter for one
            kernel, and the derived figures (clock, MFMA busy, address-unit busy, L2 hit
            rate, LDS bank conflicts) wherever the counters for them were collected
  traffic   a FETCH_SIZE and a WRITE_SIZE --pmc CSV -> bytes per dispatch per kernel,
            scaled by the copy calibration (fetch_scale, write_scale)

Every summary begins with the command lines that produced its inputs (given with
--command, one per pass), so that it can be regenerated from committed files.  Only
the standard library is used.

Examples:
  python3 bench_profile.py trace run_kernel_trace.csv --title "..." --command "rocprofv3 ..."
  python3 bench_profile.py counters idxA=a.csv idxB=b.csv --kernel indexer_prefill --kernel-source indexer
  python3 bench_profile.py traffic fetch.csv write.csv --calib profiles/copy_calibration.txt --kernel indexer_prefill
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "dsa_lightning_indexer_scores_amd", "csrc")
SOURCES = {"indexer": "indexer.hip", "topk": "topk.hip", "attention": "attn.hip", "distill": "distill.hip",
           "probe": "mfma_probe.hip"}
N_XCD, N_CU, N_SIMD = 8, 256, 1024


def source_hash(kernel: str) -> str:
    """sha256 of the kernel's source file and the shared header, as bench.py checks it."""
    h = hashlib.sha256()
    for name in (SOURCES[kernel], "common.h"):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def short_name(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("void ", "", 1)
    m = re.match(r"([\w:]+(?:<[^()]*>)?)", name)
    return (m.group(1) if m else name)[:60]


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def cmd_trace(a):
    rows = _rows(a.csv)
    by = collections.defaultdict(list)
    grid = collections.defaultdict(list)
    for r in rows:
        n = short_name(r["Kernel_Name"])
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        by[n].append(d)
        if any(g in n for g in a.grid):
            wx = int(r["Workgroup_Size_X"]) or 1
            gx = int(r["Grid_Size_X"]) // wx
            gy = int(r["Grid_Size_Y"]) // max(1, int(r["Workgroup_Size_Y"]))
            grid[(n, f"{gx}x{gy}")].append(d)
    total = sum(sum(v) for v in by.values())
    out = [f"# rocprofv3 kernel-trace summary: {a.title}"]
    out += [f"# command: {c}" for c in a.command]
    out += [f"# {x}" for x in a.note]
    # the kernel sources the trace was taken on (bench.py reads a figure only while they match)
    out += [f"source_sha256.{k}: {source_hash(k)}" for k in a.kernel_source]
    out.append("")
    out.append(f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'total_ms':>10s} {'pct':>6s}")
    for n, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"{n:60s} {len(v):6d} {sum(v) / len(v):10.1f} {min(v):10.1f} {max(v):10.1f} "
                   f"{sum(v) / 1000:10.2f} {100 * sum(v) / total:6.2f}")
    if grid:
        out.append("")
        out.append("# by launch grid (workgroups x, y)")
        out.append(f"{'kernel':60s} {'grid':>12s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}")
        for (n, g), v in sorted(grid.items()):
            out.append(f"{n:60s} {g:>12s} {len(v):6d} {sum(v) / len(v):10.1f} {min(v):10.1f} {max(v):10.1f}")
    print("\n".join(out))


def _pmc_means(path, kernel_sub):
    """Mean per dispatch of every counter of the dispatches whose kernel name contains kernel_sub,
    plus the mean duration in us and the dispatch count."""
    rows = _rows(path)
    per = collections.defaultdict(dict)
    dur = {}
    name = None
    for r in rows:
        if kernel_sub not in r["Kernel_Name"]:
            continue
        name = short_name(r["Kernel_Name"])
        did = r["Dispatch_Id"]
        c = r["Counter_Name"]
        per[did][c] = per[did].get(c, 0.0) + float(r["Counter_Value"])
        if "Start_Timestamp" in r and r.get("End_Timestamp"):
            dur[did] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
    if not per:
        raise SystemExit(f"no dispatch of a kernel containing {kernel_sub!r} in {path}")
    counters = sorted({c for d in per.values() for c in d})
    means = {c: sum(d.get(c, 0.0) for d in per.values()) / len(per) for c in counters}
    mean_dur = sum(dur.values()) / len(dur) if dur else None
    return name, means, mean_dur, len(per)


def cmd_counters(a):
    out = [f"# rocprofv3 counters: {a.title}"]
    out.append("# commands (one run per pass):")
    out += [f"#   {c}" for c in a.command]
    out.append("# values are the mean per dispatch; GRBM_GUI_ACTIVE is summed over the 8 XCDs (per-XCD cycles ="
               " value / 8); per-SQ counters are summed over the chip")
    out += [f"# {x}" for x in a.note]
    allv, durs, name = {}, [], None
    body = []
    for spec in a.passes:
        tag, path = spec.split("=", 1)
        name, means, d, n = _pmc_means(path, a.kernel)
        if d:
            durs.append(d)
        body.append(f"# pass {tag}: {n} dispatches, mean duration under the profiler "
                    f"{d:.1f} us" if d else f"# pass {tag}: {n} dispatches")
        for c, v in means.items():
            body.append(f"{tag}.{c}: {v:.6g}")
            allv.setdefault(c, v)
            allv[f"{tag}.GRBM_GUI_ACTIVE"] = means.get("GRBM_GUI_ACTIVE", 0.0)
    out.append(f"kernel: {name}")
    if a.kernel_source:
        out.append(f"source_sha256: {source_hash(a.kernel_source)}")
    out += body
    dur = sum(durs) / len(durs) if durs else None
    xcd_cycles = allv.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD
    out.append("# derived (plain keys, read by bench.py)")
    if dur and xcd_cycles:
        out.append(f"duration_us: {dur:.1f}")
        if dur >= 100.0:
            out.append(f"# clock = GRBM_GUI_ACTIVE / 8 / duration")
            out.append(f"clock_ghz: {xcd_cycles / (dur * 1e3):.3f}")
        else:
            out.append("# no clock: GRBM_GUI_ACTIVE also counts the dispatch around a kernel this short")
    if xcd_cycles:
        if "SQ_VALU_MFMA_BUSY_CYCLES" in allv:
            out.append("# mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (per-XCD cycles * 1024 SIMDs) (rocprofv3 MfmaUtil)")
            out.append(f"mfma_busy: {allv['SQ_VALU_MFMA_BUSY_CYCLES'] / (xcd_cycles * N_SIMD):.3f}")
            if "SQ_INSTS_MFMA" in allv and allv["SQ_INSTS_MFMA"]:
                out.append(f"mfma_busy_cycles_per_instruction: "
                           f"{allv['SQ_VALU_MFMA_BUSY_CYCLES'] / allv['SQ_INSTS_MFMA']:.2f}")
        if "TA_TA_BUSY_sum" in allv:
            out.append("# address_unit_busy = TA_TA_BUSY_sum / 256 / per-XCD cycles")
            out.append(f"address_unit_busy: {allv['TA_TA_BUSY_sum'] / N_CU / xcd_cycles:.3f}")
        if "SQ_LDS_BANK_CONFLICT" in allv:
            out.append("# lds_bank_conflict = SQ_LDS_BANK_CONFLICT / per-XCD cycles / 256 CUs (rocprofv3 LDSBankConflict)")
            out.append(f"lds_bank_conflict: {allv['SQ_LDS_BANK_CONFLICT'] / xcd_cycles / N_CU:.4f}")
        if "SQ_BUSY_CYCLES" in allv:
            out.append(f"sq_busy: {allv['SQ_BUSY_CYCLES'] / xcd_cycles / N_XCD:.3f}")
    if allv.get("SQ_WAVE_CYCLES"):
        fracs = [(k, c) for k, c in (("wave_wait_any_frac", "SQ_WAIT_ANY"), ("wave_wait_inst_any_frac", "SQ_WAIT_INST_ANY"),
                                     ("wave_valu_active_frac", "SQ_ACTIVE_INST_VALU"),
                                     ("wave_lds_active_frac", "SQ_ACTIVE_INST_LDS")) if c in allv]
        if fracs:
            out.append("# fractions of the waves' resident cycles (SQ_WAVE_CYCLES): waiting (on a dependency or a"
                       " barrier), waiting to issue, and issuing VALU or LDS work")
        for key, c in fracs:
            out.append(f"{key}: {allv[c] / allv['SQ_WAVE_CYCLES']:.3f}")
    if "TA_TA_BUSY_sum" in allv and "TA_FLAT_READ_WAVEFRONTS_sum" in allv and allv["TA_FLAT_READ_WAVEFRONTS_sum"]:
        out.append(f"address_unit_cycles_per_load_instruction: "
                   f"{allv['TA_TA_BUSY_sum'] / allv['TA_FLAT_READ_WAVEFRONTS_sum']:.2f}")
    if "TCC_HIT_sum" in allv and "TCC_MISS_sum" in allv:
        h, m = allv["TCC_HIT_sum"], allv["TCC_MISS_sum"]
        out.append(f"l2_hit_rate: {h / max(h + m, 1.0):.3f}")
    if "SQ_INSTS_VALU" in allv and "SQ_INSTS_MFMA" in allv and allv["SQ_INSTS_MFMA"]:
        out.append(f"valu_instructions_per_mfma: {allv['SQ_INSTS_VALU'] / allv['SQ_INSTS_MFMA']:.2f}")
    print("\n".join(out))


def _calib(path):
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = float(v.split("#")[0].strip())
    return vals["fetch_scale"], vals["write_scale"]


def cmd_traffic(a):
    fs, ws = _calib(a.calib) if a.calib else (1.0, 1.0)
    fr = collections.defaultdict(list)
    wr = collections.defaultdict(list)
    for path, store, cname in ((a.fetch, fr, "FETCH_SIZE"), (a.write, wr, "WRITE_SIZE")):
        per = collections.defaultdict(float)
        names = {}
        for r in _rows(path):
            if r["Counter_Name"] != cname:
                continue
            per[r["Dispatch_Id"]] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = short_name(r["Kernel_Name"])
        for did, v in per.items():
            store[names[did]].append(v)
    out = [f"# HBM traffic per dispatch from FETCH_SIZE / WRITE_SIZE: {a.title}"]
    out += [f"# command: {c}" for c in a.command]
    out.append(f"# bytes = counter KiB * 1024 * scale (copy calibration: fetch_scale {fs:.4f}, write_scale {ws:.4f})")
    out += [f"# {x}" for x in a.note]
    if a.kernel_source:
        out.append(f"source_sha256: {source_hash(a.kernel_source)}")
    out.append(f"{'kernel':60s} {'dispatches':>10s} {'fetch_KiB':>12s} {'write_KiB':>12s} {'read_MB':>10s} {'write_MB':>10s}")
    for n in sorted(set(fr) | set(wr)):
        f = fr.get(n, [0.0])
        w = wr.get(n, [0.0])
        fk, wk = sum(f) / len(f), sum(w) / len(w)
        out.append(f"{n:60s} {max(len(f), len(w)):10d} {fk:12.1f} {wk:12.1f} {fk * 1024 * fs / 1e6:10.2f} "
                   f"{wk * 1024 * ws / 1e6:10.2f}")
    if a.kernel:
        sel = [n for n in set(fr) | set(wr) if a.kernel in n]
        if sel:
            n = sel[0]
            fk = sum(fr.get(n, [0.0])) / max(1, len(fr.get(n, [0.0])))
            wk = sum(wr.get(n, [0.0])) / max(1, len(wr.get(n, [0.0])))
            out.append(f"kernel: {n}")
            out.append(f"fetch_size_kib_per_dispatch: {fk:.1f}")
            out.append(f"write_size_kib_per_dispatch: {wk:.1f}")
            out.append(f"traffic_bytes_per_launch: {(fk * fs + wk * ws) * 1024:.6g}")
    print("\n".join(out))


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = p.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("csv")
    t.add_argument("--grid", action="append", default=[])
    t.add_argument("--kernel-source", action="append", default=[], choices=sorted(SOURCES))
    c = sub.add_parser("counters")
    c.add_argument("passes", nargs="+", help="TAG=counter_collection.csv, one per pass")
    c.add_argument("--kernel", required=True, help="substring of the kernel name")
    c.add_argument("--kernel-source", choices=sorted(SOURCES), default=None)
    f = sub.add_parser("traffic")
    f.add_argument("fetch")
    f.add_argument("write")
    f.add_argument("--calib", default=None)
    f.add_argument("--kernel", default=None)
    f.add_argument("--kernel-source", choices=sorted(SOURCES), default=None)
    for s in (t, c, f):
        s.add_argument("--title", default="")
        s.add_argument("--command", action="append", default=[])
        s.add_argument("--note", action="append", default=[])
    a = p.parse_args(argv)
    {"trace": cmd_trace, "counters": cmd_counters, "traffic": cmd_traffic}[a.cmd](a)


if __name__ == "__main__":
    main()
