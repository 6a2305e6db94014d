"""Summaries of rocprofv3 output for the library's kernels.

    python -m w4a4_quantized_linear_cube_amd.profiling trace DIR OUT.md CMD...
        kernel-trace statistics (DIR/*_kernel_stats.csv) -> markdown table
    python -m w4a4_quantized_linear_cube_amd.profiling counters RUN_FETCH RUN_WRITE COPY_FETCH COPY_WRITE
            --copy-bytes B --config NAME --cube t,h,w --out OUT.json --cmd "..."
        FETCH_SIZE / WRITE_SIZE per dispatch of the delta GEMM, each scaled by
        the same counter's reading for plain device copies of known size
        (B bytes read and B bytes written in total), -> HBM bytes per launch

The counter JSON records the SHA-256 of gemm.hip; bench.py reports its
traffic only while the kernel source is unchanged.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
DELTA_KERNEL = re.compile(r"k_gemm<4, [12], ")     # the delta GEMM (FP4 B operand, token epilogue)
CORE_KERNEL = re.compile(r"k_gemm<0, 0, ")
COPY_KERNEL = re.compile(r"copyBuffer")


def _short(name: str) -> str:
    return re.sub(r"\(.*", "", name)


def summarize_trace(d: str, out: str, cmd: str) -> None:
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    rows = list(csv.DictReader(open(files[0])))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    # Per-dispatch durations (DIR/*_kernel_trace.csv) give the median, which
    # the first dispatches (clock still ramping) do not move.
    durs = defaultdict(list)
    for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            durs[r["Kernel_Name"]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))

    def median_us(name):
        v = sorted(durs.get(name, []))
        return f"{v[len(v) // 2] / 1e3:.1f}" if v else "-"

    lines = ["# Kernel trace: " + os.path.splitext(os.path.basename(out))[0], "",
             "Command (from the repository root on the GPU box):", "", "```", cmd, "```", "",
             "| kernel | calls | average (us) | median (us) | min (us) | max (us) | total (ms) |",
             "|---|---|---|---|---|---|---|"]
    for r in rows[:12]:
        lines.append(f"| `{_short(r['Name'])[:70]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{median_us(r['Name'])} | {float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.2f} |")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter_per_dispatch(d: str, counter: str, pattern) -> list:
    """Sum of `counter` over the instances of each matching dispatch."""
    per = defaultdict(float)
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter or not pattern.search(r["Kernel_Name"]):
                continue
            per[(f, r["Dispatch_Id"])] += float(r["Counter_Value"])
    return list(per.values())


def summarize_counters(run_fetch, run_write, copy_fetch, copy_write, copy_bytes, config, cube, out, cmd):
    df = _counter_per_dispatch(run_fetch, "FETCH_SIZE", DELTA_KERNEL)
    dw = _counter_per_dispatch(run_write, "WRITE_SIZE", DELTA_KERNEL)
    cf = _counter_per_dispatch(copy_fetch, "FETCH_SIZE", COPY_KERNEL)
    cw = _counter_per_dispatch(copy_write, "WRITE_SIZE", COPY_KERNEL)
    if not (df and dw and cf and cw):
        raise SystemExit("missing dispatches: delta GEMM %d/%d, copy %d/%d" % (len(df), len(dw), len(cf), len(cw)))
    fetch_kib, write_kib = sum(df) / len(df), sum(dw) / len(dw)
    f_scale = copy_bytes / (sum(cf) * 1024.0)      # true bytes per counted byte
    w_scale = copy_bytes / (sum(cw) * 1024.0)
    fetch_b, write_b = fetch_kib * 1024 * f_scale, write_kib * 1024 * w_scale
    src = os.path.join(HERE, "csrc", "gemm.hip")
    rec = {
        "kernel": "delta GEMM (k_gemm, FP4 B operand, token epilogue)",
        "config": config, "cube": list(cube),
        "dispatches": {"fetch": len(df), "write": len(dw)},
        "fetch_kib_per_dispatch": round(fetch_kib, 1), "write_kib_per_dispatch": round(write_kib, 1),
        "copy_calibration": {"bytes_each_way": copy_bytes, "fetch_kib": round(sum(cf), 1),
                             "write_kib": round(sum(cw), 1), "fetch_scale": round(f_scale, 4),
                             "write_scale": round(w_scale, 4)},
        "fetch_bytes": int(fetch_b), "write_bytes": int(write_b), "traffic_bytes": int(fetch_b + write_b),
        "gemm_hip_sha256": hashlib.sha256(open(src, "rb").read()).hexdigest(),
        "command": cmd,
    }
    json.dump(rec, open(out, "w"), indent=1)
    print(json.dumps(rec, indent=1))


def main(argv):
    if len(argv) >= 4 and argv[0] == "trace":
        summarize_trace(argv[1], argv[2], " ".join(argv[3:]))
        return
    if argv and argv[0] == "counters":
        import argparse
        ap = argparse.ArgumentParser()
        ap.add_argument("dirs", nargs=4)
        ap.add_argument("--copy-bytes", type=int, required=True)
        ap.add_argument("--config", required=True)
        ap.add_argument("--cube", required=True)
        ap.add_argument("--out", required=True)
        ap.add_argument("--cmd", required=True)
        a = ap.parse_args(argv[1:])
        summarize_counters(*a.dirs, a.copy_bytes, a.config, [int(v) for v in a.cube.split(",")], a.out, a.cmd)
        return
    raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
