"""Summaries of rocprofv3 output for the benchmark's kernels (host tool; it
never touches the GPU).

    # kernel durations (from `rocprofv3 --kernel-trace --stats -f csv`)
    python -m flashattention_paged_kv_amd.profiling stats KT_kernel_stats.csv \\
        --cmd "<the rocprofv3 command>" --title "..." --out profiles/<name>.md
    # the same per (kernel, grid) from the kernel trace itself
    python -m flashattention_paged_kv_amd.profiling trace KT_kernel_trace.csv \\
        --cmd "<the rocprofv3 command>" --title "..." --out profiles/<name>.md

    # HBM traffic per launch (from `rocprofv3 --pmc FETCH_SIZE` and
    # `--pmc WRITE_SIZE` runs of the benchmark and of its copy calibration)
    python -m flashattention_paged_kv_amd.profiling traffic \\
        --fetch F.csv --write W.csv --copy-fetch CF.csv --copy-write CW.csv \\
        --copy-bytes N --kernel decode_split_kernel --out profiles/traffic.json

FETCH_SIZE / WRITE_SIZE are read in KiB per dispatch.  On a partitioned
device they need not see every memory channel, so each is scaled by the
ratio known-bytes / counter for a plain device copy of N bytes (the
`__amd_rocclr_copyBuffer` dispatches of `bench.py --copy-calibration N`).
The traffic file records a hash of the kernel's sources; `bench.py` only
reports traffic while the sources are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
import sys
from collections import defaultdict

_HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(_HERE, "csrc")

# Kernel name fragment -> source files whose text defines it.
KERNEL_SOURCES = {
    "prefill_bf16_kernel": ("prefill.hip", "pa_device.h", "pa_internal.h"),
    # the same kernel with the append fused in (its 4th template argument)
    "prefill_bf16_kernel_fused": ("prefill.hip", "pa_device.h", "pa_internal.h"),
    "decode_split_kernel": ("decode.hip", "pa_device.h", "pa_internal.h"),
    "decode_reduce_kernel": ("decode.hip", "pa_device.h", "pa_internal.h"),
    "append_kernel": ("append.hip", "pa_device.h", "pa_internal.h"),
}


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    for k in KERNEL_SOURCES:
        if k in name:
            return name.split("(")[0].replace("void ", "")
    return name if len(name) <= 60 else name[:57] + "..."


def stats_markdown(stats_csv: str, cmd: str, title: str) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    out = [f"# {title}", "", "Command (from the repository root, on one MI355X):", "", "```", cmd, "```", "",
           "| kernel | calls | avg µs | min µs | max µs |", "|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    return "\n".join(out) + "\n"


def trace_markdown(trace_csv: str, cmd: str, title: str, min_calls: int = 1) -> str:
    """Per (kernel, grid) launch statistics from a `--kernel-trace` CSV: one
    kernel instantiation launched with different grids (the same prefill
    kernel at 2k and at 32k rows) gets one row per grid.  Grid sizes are in
    work items, as rocprofv3 reports them."""
    groups = defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        grid = (int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]), int(r["Grid_Size_Z"]))
        groups[(_short(r["Kernel_Name"]), grid)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = [f"# {title}", "", "Command (from the repository root, on one MI355X):", "", "```", cmd, "```", "",
           "| kernel | grid (work items) | calls | avg µs | median µs | min µs | max µs |",
           "|---|---|---|---|---|---|---|"]
    rows = sorted(groups.items(), key=lambda kv: -sum(kv[1]))
    for (name, grid), d in rows:
        if len(d) < min_calls:
            continue
        out.append(f"| `{name}` | {grid[0]}×{grid[1]}×{grid[2]} | {len(d)} | {statistics.fmean(d):.1f} | "
                   f"{statistics.median(d):.1f} | {min(d):.1f} | {max(d):.1f} |")
    return "\n".join(out) + "\n"


def pmc_markdown(paths, cmds, title: str, simds: int, xccs: int, match: str = "") -> str:
    """Counters per dispatch, averaged per (kernel, grid), from one or more
    `rocprofv3 --pmc` runs (one counter set each), with the MFMA utilisation
    they give and the bf16 MFMA work executed (SQ_INSTS_VALU_MFMA_MOPS_BF16 x
    512 FLOPs).

    SQ_VALU_MFMA_BUSY_CYCLES arrives summed over every SIMD of the device
    (for v_mfma_f32_32x32x16_bf16 it equals 32 cycles x the MFMAs executed),
    GRBM_GUI_ACTIVE summed over the XCDs (each counts the cycles its XCD was
    busy), so the utilisation is busy / (SIMDs x GRBM_GUI_ACTIVE / XCDs):
    rocprofv3's own MfmaUtil expression, which takes the largest XCD's count
    instead of the sum.  The shader clock implied by GRBM_GUI_ACTIVE / XCDs
    over the dispatch's duration is shown beside it."""
    vals = defaultdict(lambda: defaultdict(list))
    durs = defaultdict(dict)
    for path in paths:
        for r in csv.DictReader(open(path)):
            if match and match not in r["Kernel_Name"]:
                continue
            key = (_short(r["Kernel_Name"]), r.get("Grid_Size", "?"))
            vals[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                durs[key][len(vals[key]["GRBM_GUI_ACTIVE"]) - 1] = (
                    float(r["Counter_Value"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = [f"# {title}", "", "Commands (from the repository root, on one MI355X; one counter set per run):", "",
           "```", *cmds, "```", "",
           f"Per dispatch, averaged over the dispatches of each (kernel, grid); {simds} SIMDs in {xccs} XCDs.", ""]
    for (name, grid), cs in sorted(vals.items()):
        out.append(f"## `{name}`, grid {grid} work items")
        out.append("")
        out.append("| counter | dispatches | mean per dispatch |")
        out.append("|---|---|---|")
        for c, v in sorted(cs.items()):
            out.append(f"| {c} | {len(v)} | {statistics.fmean(v):.6g} |")
        m = {c: statistics.fmean(v) for c, v in cs.items()}
        if "GRBM_GUI_ACTIVE" in m and durs[(name, grid)]:
            ghz = statistics.fmean(g / xccs / max(1, d) for g, d in durs[(name, grid)].values())
            out.append(f"| shader clock implied (GRBM_GUI_ACTIVE / XCDs / duration) | | {ghz:.2f} GHz |")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m and "GRBM_GUI_ACTIVE" in m and m["GRBM_GUI_ACTIVE"] > 0:
            out.append(f"| **MFMA utilisation** (busy / (SIMDs x GRBM_GUI_ACTIVE / XCDs)) | | "
                       f"**{100 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / (m['GRBM_GUI_ACTIVE'] / xccs * simds):.1f}%** |")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m and durs[(name, grid)]:
            dur_ns = statistics.fmean(d for _, d in durs[(name, grid)].values())
            out.append(f"| MFMA busy / (SIMDs x dispatch duration x 2.4 GHz): share of the nominal peak | | "
                       f"{100 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / simds / (dur_ns * 2.4):.1f}% "
                       f"(duration {dur_ns / 1e3:.1f} µs) |")
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in m:
            out.append(f"| bf16 MFMA FLOPs executed (MOPS x 512) | | {m['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512:.6g} |")
        out.append("")
    return "\n".join(out)


def counter_per_dispatch(path: str, counter: str) -> dict:
    """Mean value of `counter` per dispatch, by kernel name."""
    vals = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: statistics.fmean(v) for k, v in vals.items()}


def _pick(d: dict, fragment: str) -> float:
    hits = [v for k, v in d.items() if fragment in k]
    if not hits:
        raise SystemExit(f"no dispatch of a kernel named like {fragment!r}")
    return statistics.fmean(hits)


def traffic(args) -> dict:
    fetch = counter_per_dispatch(args.fetch, "FETCH_SIZE")
    write = counter_per_dispatch(args.write, "WRITE_SIZE")
    cfetch = _pick(counter_per_dispatch(args.copy_fetch, "FETCH_SIZE"), "copyBuffer")
    cwrite = _pick(counter_per_dispatch(args.copy_write, "WRITE_SIZE"), "copyBuffer")
    f_scale = args.copy_bytes / (cfetch * 1024.0)
    w_scale = args.copy_bytes / (cwrite * 1024.0)
    match = args.match or args.kernel
    rd = _pick(fetch, match) * 1024.0 * f_scale
    wr = _pick(write, match) * 1024.0 * w_scale
    return dict(kernel=args.kernel, match=match, source_hash=source_hash(args.kernel), workload=args.workload,
                read_bytes_per_launch=rd, write_bytes_per_launch=wr, hbm_bytes_per_launch=rd + wr,
                fetch_scale=f_scale, write_scale=w_scale, copy_bytes=args.copy_bytes)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(prog="python -m flashattention_paged_kv_amd.profiling")
    sub = ap.add_subparsers(dest="action", required=True)
    s = sub.add_parser("stats")
    s.add_argument("stats_csv")
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--out", required=True)
    k = sub.add_parser("trace")
    k.add_argument("trace_csv")
    k.add_argument("--cmd", required=True)
    k.add_argument("--title", required=True)
    k.add_argument("--out", required=True)
    k.add_argument("--min-calls", type=int, default=1)
    pm = sub.add_parser("pmc")
    pm.add_argument("csv", nargs="+", help="counter_collection.csv of each --pmc run")
    pm.add_argument("--cmd", action="append", required=True, help="the rocprofv3 command of each run")
    pm.add_argument("--title", required=True)
    pm.add_argument("--simds", type=int, default=1024, help="SIMDs of the device (MI355X: 256 CUs x 4)")
    pm.add_argument("--xccs", type=int, default=8, help="XCDs of the device (MI355X: 8)")
    pm.add_argument("--match", default="", help="only kernels whose name contains this")
    pm.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    for n in ("fetch", "write", "copy-fetch", "copy-write"):
        t.add_argument("--" + n, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--kernel", required=True, choices=sorted(KERNEL_SOURCES))
    t.add_argument("--match", default=None,
                   help="kernel-name fragment to select dispatches by (default: --kernel), e.g. "
                        "'prefill_bf16_kernel<128, true, false, true>' for one instantiation")
    t.add_argument("--workload", required=True)
    t.add_argument("--out", required=True)
    args = ap.parse_args(argv)
    if args.action == "pmc":
        with open(args.out, "w") as f:
            f.write(pmc_markdown(args.csv, args.cmd, args.title, args.simds, args.xccs, args.match))
        return 0
    if args.action == "trace":
        with open(args.out, "w") as f:
            f.write(trace_markdown(args.trace_csv, args.cmd, args.title, args.min_calls))
        return 0
    if args.action == "stats":
        with open(args.out, "w") as f:
            f.write(stats_markdown(args.stats_csv, args.cmd, args.title))
        return 0
    rec = traffic(args)
    data = {}
    if os.path.exists(args.out):
        with open(args.out) as f:
            data = json.load(f)
    data[f"{args.kernel}:{args.workload}"] = rec
    with open(args.out, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main())
