"""Summaries of rocprofv3 output for the profiles/ folder.

    # per-kernel durations (from a --kernel-trace --stats run)
    python -m lora_bypass_linear_amd.profsum stats DIR --cmd "<command>" --out profiles/NAME.txt

    # MFMA busy fraction and MFMA flops of one kernel (one --pmc run)
    python -m lora_bypass_linear_amd.profsum mfma DIR --kernel SUBSTR --cmd "<command>" --out profiles/NAME.txt

    # HBM traffic of one kernel (from one --pmc FETCH_SIZE run and one --pmc
    # WRITE_SIZE run of a command that also performs a plain copy of a known size)
    python -m lora_bypass_linear_amd.profsum traffic --fetch DIR_F --write DIR_W --kernel SUBSTR \\
        --sources gemm|hpass|merge --calib-kernel copyBuffer --calib-bytes N --cmd "<commands>" --out profiles/NAME.txt

FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch.  Each is scaled by
the ratio (known bytes of the copy) / (what the same counter reports for the
copy kernel), so the figures are bytes as the copy kernel defines them.  The
traffic summary records a hash of the profiled kernel's sources; bench.py uses
the figure only while the sources still hash to it.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
# the sources each profiled kernel is built from
SOURCES = {"gemm": ("csrc/gemm.hip", "csrc/kernels.h", "csrc/lyc_device.h"),
           "hpass": ("csrc/hpass.hip", "csrc/kernels.h", "csrc/lyc_device.h"),
           "merge": ("csrc/merge.hip", "csrc/merge.h", "csrc/lyc_device.h")}


def source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for rel in SOURCES[kind]:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _find(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[0]


def stats(args) -> str:
    path = _find(args.dir, "kernel_stats.csv")
    rows = list(csv.DictReader(open(path)))
    lines = [f"# rocprofv3 kernel statistics", f"command: {args.cmd}", "",
             f"{'kernel':<100} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_%':>8}"]
    for r in rows:
        name = r["Name"].strip('"')
        lines.append(f"{name[:100]:<100} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} "
                     f"{float(r['MinNs']) / 1e3:>10.2f} {float(r['MaxNs']) / 1e3:>10.2f} {float(r['Percentage']):>8.2f}")
    return "\n".join(lines) + "\n"


def _per_dispatch(path: str, counter: str):
    """{dispatch id: (kernel name, value summed over the counter's instances)}"""
    out = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        name, v = out.get(d, (r["Kernel_Name"], 0.0))
        out[d] = (name, v + float(r["Counter_Value"]))
    return out


def traffic(args) -> str:
    res = {}
    for tag, d, counter in (("fetch", args.fetch, "FETCH_SIZE"), ("write", args.write, "WRITE_SIZE")):
        per = _per_dispatch(_find(d, "counter_collection.csv"), counter)
        cal = [v for n, v in per.values() if args.calib_kernel in n]
        ker = [v for n, v in per.values() if args.kernel in n]
        if not cal or not ker:
            raise SystemExit(f"{counter}: calibration kernel or kernel not found in {d}")
        factor = args.calib_bytes / (max(cal) * 1024.0)
        res[tag] = (statistics.median(ker) * 1024.0 * factor, factor, len(ker), statistics.median(ker))
    lines = ["# HBM traffic per launch (rocprofv3 --pmc FETCH_SIZE, --pmc WRITE_SIZE)",
             f"command: {args.cmd}",
             f"kernel: {args.kernel}",
             f"sources: {args.sources}",
             f"source_sha: {source_hash(args.sources)}",
             f"calibration: plain copy kernel '{args.calib_kernel}' of {args.calib_bytes} bytes",
             f"fetch_factor: {res['fetch'][1]:.4f}",
             f"write_factor: {res['write'][1]:.4f}",
             f"fetch_kib_raw_median: {res['fetch'][3]:.1f}",
             f"write_kib_raw_median: {res['write'][3]:.1f}",
             f"dispatches: {res['fetch'][2]}",
             f"fetch_bytes_per_launch: {res['fetch'][0]:.0f}",
             f"write_bytes_per_launch: {res['write'][0]:.0f}",
             f"traffic_bytes_per_launch: {res['fetch'][0] + res['write'][0]:.0f}"]
    return "\n".join(lines) + "\n"


def mfma(args) -> str:
    """MFMA activity of one kernel from a --pmc run of SQ_VALU_MFMA_BUSY_CYCLES,
    SQ_INSTS_VALU_MFMA_MOPS_F16, SQ_INSTS_VALU_MFMA_MOPS_BF16 and GRBM_GUI_ACTIVE:
    the fraction of SIMD cycles in which the matrix pipe was busy while the
    GPU was active, and the MFMA flops the counters saw (MOPS count units of
    512 flops).  GRBM_GUI_ACTIVE is counted once per XCD (the value is the
    sum over the XCDs' instances), SQ_VALU_MFMA_BUSY_CYCLES once per SIMD."""
    path = _find(args.dir, "counter_collection.csv")
    vals = {}
    for c in ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
              "GRBM_GUI_ACTIVE"):
        per = _per_dispatch(path, c)
        ker = [v for n, v in per.values() if args.kernel in n]
        if not ker:
            raise SystemExit(f"{c}: kernel not found in {args.dir}")
        vals[c] = statistics.median(ker)
    busy, active = vals["SQ_VALU_MFMA_BUSY_CYCLES"], vals["GRBM_GUI_ACTIVE"] / args.xcds
    flops = (vals["SQ_INSTS_VALU_MFMA_MOPS_F16"] + vals["SQ_INSTS_VALU_MFMA_MOPS_BF16"]) * 512.0
    lines = ["# MFMA activity per launch (rocprofv3 --pmc, median over dispatches)",
             f"command: {args.cmd}",
             f"kernel: {args.kernel}",
             f"simds: {args.simds}",
             f"xcds: {args.xcds}",
             f"mfma_busy_cycles: {busy:.0f}",
             f"gui_active_cycles_per_xcd: {active:.0f}",
             f"mfma_busy_fraction: {busy / max(active * args.simds, 1.0):.4f}",
             f"mfma_flops_per_launch: {flops:.6g}"]
    return "\n".join(lines) + "\n"


def read_traffic(path: str, kind: str):
    """traffic bytes per launch from a summary, or None if it is missing or stale."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("sources") != kind or kv.get("source_sha") != source_hash(kind):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--cmd", required=True)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--sources", required=True, choices=sorted(SOURCES))
    t.add_argument("--calib-kernel", required=True)
    t.add_argument("--calib-bytes", type=float, required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--out", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("dir")
    m.add_argument("--kernel", required=True)
    m.add_argument("--simds", type=int, default=1024)
    m.add_argument("--xcds", type=int, default=8)
    m.add_argument("--cmd", required=True)
    m.add_argument("--out", required=True)
    args = ap.parse_args(argv)
    text = {"stats": stats, "traffic": traffic, "mfma": mfma}[args.mode](args)
    os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
    with open(args.out, "w") as f:
        f.write(text)
    sys.stdout.write(text)


if __name__ == "__main__":
    main()
