"""Summaries of rocprofv3 output for the dMoE kernels.

    python -m dropless_mixture_experts_amd.profiling stats DIR [--window S:N]
        Per-kernel call count, total and average duration from the
        kernel-trace CSV under DIR (rocprofv3 --kernel-trace --stats
        --output-format csv).  --window S:N adds the average over each
        kernel's calls S .. S+N-1 in launch order (e.g. a benchmark's timed
        steps, without its warm-up and untimed passes).

    python -m dropless_mixture_experts_amd.profiling traffic \\
        --fetch DIR_F --write DIR_W --kernel REGEX --name BENCH_NAME \\
        --workload NAME \\
        --copy-bytes N [--copy-kernel REGEX] [--source FILE] --out JSON
        HBM traffic per launch of the kernels matching REGEX from two
        counter runs (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch).
        Each counter is scaled by what it reads for a plain copy kernel of
        N bytes in the same run (bytes read = bytes written = N), so the
        factor corrects whatever unit or sampling the counter has.  The
        sha256 of --source is stored so that a later change of the kernel
        makes the figure stale.

    python -m dropless_mixture_experts_amd.profiling counters \
        --kernel NAME=REGEX [--kernel ...] DIR [DIR ...]
        Medians over dispatches of every counter found in the counter CSVs
        under the DIRs (one rocprofv3 --pmc pass each), per kernel, and the
        derived figures: mfma = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE
        * 128) (GRBM_GUI_ACTIVE is summed over 8 XCDs of 128 SIMDs each),
        clock_ghz = GRBM_GUI_ACTIVE / (8 * dispatch duration) (the
        effective shader clock; needs the rows' timestamps),
        l2hit = TCC_HIT / (TCC_HIT + TCC_MISS), ta = TA_TA_BUSY /
        (GRBM_GUI_ACTIVE * 32) and tcp = TCP_PENDING_STALL_CYCLES /
        (GRBM_GUI_ACTIVE * 32) (32 CUs per XCD), and mfma_gflop =
        SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512 / 1e9, the matrix-core work of one
        launch.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys


def _rows(directory: str, pattern: str):
    files = glob.glob(os.path.join(directory, "**", pattern), recursive=True)
    out = []
    for f in sorted(files):
        with open(f) as fh:
            out.extend(csv.DictReader(fh))
    return out


def kernel_durations(directory: str):
    """{kernel name: [duration_ns, ...] in launch order} from a kernel-trace CSV."""
    rows = _rows(directory, "*kernel_trace.csv")
    acc = {}
    for r in rows:
        name = r.get("Kernel_Name") or r.get("KernelName")
        start = int(r["Start_Timestamp"])
        acc.setdefault(name, []).append((start, int(r["End_Timestamp"]) - start))
    return {k: [d for _, d in sorted(v)] for k, v in acc.items()}


def kernel_stats(directory: str):
    """{kernel name: (calls, total_ns, avg_ns)} from a kernel-trace CSV."""
    return {k: (len(v), sum(v), sum(v) / len(v)) for k, v in kernel_durations(directory).items()}


def _counter(directory: str, counter: str, kernel_re: str):
    vals = []
    for r in _rows(directory, "*counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        if re.search(kernel_re, r["Kernel_Name"]):
            vals.append(float(r["Counter_Value"]))
    return vals


def counter_medians(dirs, kernels):
    """{name: {counter: median over dispatches}} for (name, regex) pairs.
    Where the rows carry dispatch timestamps, "clock_ghz" is the median over
    dispatches of GRBM_GUI_ACTIVE / (8 * duration): the effective shader
    clock while the kernel ran (GRBM_GUI_ACTIVE counts busy cycles of each
    of the 8 XCDs and sums them)."""
    rows = [r for d in dirs for r in _rows(d, "*counter_collection.csv")]
    out = {}
    for name, rx in kernels:
        per = {}
        clk = []
        for r in rows:
            if re.search(rx, r["Kernel_Name"]):
                per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                if r["Counter_Name"] == "GRBM_GUI_ACTIVE" and r.get("Start_Timestamp"):
                    ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                    if ns > 0:
                        clk.append(float(r["Counter_Value"]) / 8.0 / ns)
        out[name] = {c: statistics.median(v) for c, v in per.items()}
        if clk:
            out[name]["clock_ghz"] = statistics.median(clk)
    return out


def derived(c: dict) -> dict:
    def ratio(num, den, scale=1.0):
        if num in c and den in c and c[den] > 0:
            return c[num] / (c[den] * scale)
        return None
    hit, miss = c.get("TCC_HIT_sum"), c.get("TCC_MISS_sum")
    return {
        "mfma": ratio("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", 128.0),
        "l2hit": hit / (hit + miss) if hit is not None and miss is not None and hit + miss > 0
        else None,
        "ta": ratio("TA_TA_BUSY_sum", "GRBM_GUI_ACTIVE", 32.0),
        "tcp": ratio("TCP_PENDING_STALL_CYCLES_sum", "GRBM_GUI_ACTIVE", 32.0),
        "lds_bankcf": c.get("SQ_LDS_BANK_CONFLICT"),
        "clock_ghz": c.get("clock_ghz"),
        # SQ_INSTS_VALU_MFMA_MOPS_BF16 counts units of 512 FLOP
        "mfma_gflop": (c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / 1e9
                       if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c else None),
    }


def traffic(args) -> dict:
    fetch = _counter(args.fetch, "FETCH_SIZE", args.kernel)
    write = _counter(args.write, "WRITE_SIZE", args.kernel)
    cf = _counter(args.fetch, "FETCH_SIZE", args.copy_kernel)
    cw = _counter(args.write, "WRITE_SIZE", args.copy_kernel)
    if not (fetch and write and cf and cw):
        raise SystemExit("missing counter rows: kernel or copy kernel not found")
    # the copy of N bytes: median dispatch, counters in KiB
    f_factor = args.copy_bytes / (statistics.median(cf) * 1024.0)
    w_factor = args.copy_bytes / (statistics.median(cw) * 1024.0)
    fetch_b = statistics.median(fetch) * 1024.0 * f_factor
    write_b = statistics.median(write) * 1024.0 * w_factor
    out = {
        "bench_name": args.name,
        "kernel_regex": args.kernel,
        "workload": args.workload,
        "fetch_kib_per_dispatch": statistics.median(fetch),
        "write_kib_per_dispatch": statistics.median(write),
        "copy_bytes": args.copy_bytes,
        "copy_fetch_kib": statistics.median(cf),
        "copy_write_kib": statistics.median(cw),
        "fetch_factor": f_factor,
        "write_factor": w_factor,
        "traffic_bytes_per_launch": fetch_b + write_b,
        "fetch_bytes_per_launch": fetch_b,
        "write_bytes_per_launch": write_b,
    }
    if args.source:
        with open(args.source, "rb") as fh:
            out["source"] = os.path.relpath(args.source)
            out["source_sha256"] = hashlib.sha256(fh.read()).hexdigest()
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--window", help="S:N, the average over calls S .. S+N-1 too")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--name", required=True, help="kernel name in bench.py's table")
    t.add_argument("--copy-kernel", default="elementwise|copy")
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--source")
    t.add_argument("--out")
    c = sub.add_parser("counters")
    c.add_argument("--kernel", action="append", required=True, help="NAME=REGEX")
    c.add_argument("dirs", nargs="+")
    a = ap.parse_args(argv)
    if a.cmd == "counters":
        kernels = [tuple(k.split("=", 1)) for k in a.kernel]
        med = counter_medians(a.dirs, kernels)
        cols = ("mfma", "l2hit", "ta", "tcp", "lds_bankcf", "mfma_gflop", "clock_ghz")
        print(f"{'kernel':28s} " + " ".join(f"{c:>10s}" for c in cols))
        for name, _ in kernels:
            d = derived(med[name])
            cells = []
            for col in cols:
                v = d[col]
                cells.append(f"{'-':>10s}" if v is None else
                             (f"{v:10.0f}" if col == "lds_bankcf" else
                              f"{v:10.2f}" if col == "mfma_gflop" else f"{v:10.3f}"))
            print(f"{name:28s} " + " ".join(cells))
        return 0
    if a.cmd == "stats":
        durs = kernel_durations(a.dir)
        win = tuple(int(v) for v in a.window.split(":")) if a.window else None
        head = f"{'kernel':72s} {'calls':>6s} {'total_us':>11s} {'avg_us':>10s}"
        print(head + (f" {'window_avg_us':>14s}" if win else ""))
        for k, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
            line = f"{k[:72]:72s} {len(v):6d} {sum(v) / 1e3:11.1f} {sum(v) / len(v) / 1e3:10.2f}"
            if win:
                w = v[win[0]:win[0] + win[1]]
                line += f" {sum(w) / len(w) / 1e3:14.2f}" if w else f" {'-':>14s}"
            print(line)
    else:
        res = traffic(a)
        text = json.dumps(res, indent=1)
        if a.out:
            with open(a.out, "w") as fh:
                fh.write(text + "\n")
        print(text)


if __name__ == "__main__":
    sys.exit(main())
