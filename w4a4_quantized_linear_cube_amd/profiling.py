"""Summaries of rocprofv3 output for the library's kernels.

    python -m w4a4_quantized_linear_cube_amd.profiling trace DIR OUT.md CMD...
        kernel-trace statistics (DIR/*_kernel_stats.csv) -> markdown table
    python -m w4a4_quantized_linear_cube_amd.profiling counters RUN_FETCH RUN_WRITE COPY_FETCH COPY_WRITE
            --copy-bytes B --config NAME --cube t,h,w --out OUT.json --cmd "..."
        FETCH_SIZE / WRITE_SIZE per dispatch of the delta GEMM (and of the
        activation pass and the core GEMM), each scaled by the same counter's
        reading for plain device copies of known size (B bytes read and B
        bytes written in total), -> HBM bytes per launch
    python -m w4a4_quantized_linear_cube_amd.profiling mfma RUN OUT.md --cmd "..."
        SQ_INSTS_VALU_MFMA_MOPS_{F6F4,F8,BF16}, SQ_VALU_MFMA_BUSY_CYCLES and
        GRBM_GUI_ACTIVE per dispatch of each kernel -> MFMA flops executed and
        MFMA utilisation (busy cycles per SIMD / active cycles per XCD)
    python -m w4a4_quantized_linear_cube_amd.profiling issue RUN OUT.md --elements E --cmd "..." [--probe F]
            [--lds RUN2 --lds-cmd "..."]
        SQ_WAVES, SQ_INSTS_{VALU,SALU,LDS} and GRBM_GUI_ACTIVE per dispatch
        -> instructions per wave, VALU issue share, VALU lane-instructions
        per activation element (E = N x Ci); F: a --stream-probe line;
        RUN2: SQ_LDS_BANK_CONFLICT per LDS instruction and per active cycle

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
# k_gemm<A format, B format, epilogue, ...>
DELTA_KERNEL = re.compile(r"k_gemm<4, 4, [12], ")          # the delta GEMM (FP4 x FP4, token epilogue)
CORE_KERNEL = re.compile(r"k_gemm<(4, [04]|16, 16), 0, ")   # the core GEMM (FP8, FP4 or bf16 cores, plain stores)
W6_KERNEL = re.compile(r"k_gemm<[23], [23], [12], ")        # the 6-bit layers' FP6 x FP6 GEMM
QUANT_KERNEL = re.compile(r"k_quantize<")
FUSED_KERNEL = re.compile(r"k_fused")                      # the one-kernel forward (core and delta in one K loop)
SIMDS = 1024                                     # 256 CUs x 4 SIMDs
CUS = 256
XCDS = 8                                         # GRBM_GUI_ACTIVE comes summed over the XCDs
COPY_KERNEL = re.compile(r"copyBuffer")


def _short(name: str) -> str:
    return re.sub(r"\(.*", "", name.replace("(anonymous namespace)::", ""))


def summarize_trace(d: str, out: str, cmd: str) -> None:
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    rows = list(csv.DictReader(open(files[0])))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    # Per-dispatch durations (DIR/*_kernel_trace.csv) give the median, which
    # the first dispatches (clock still ramping) do not move.
    durs = defaultdict(list)
    shapes = defaultdict(list)                   # (library kernel, grid) -> durations
    for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            durs[r["Kernel_Name"]].append(ns)
            if "dq::" in r["Kernel_Name"]:
                grid = r.get("Grid_Size_X") or r.get("Grid_Size") or "?"
                shapes[(r["Kernel_Name"], grid)].append(ns)

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
    # every launch shape of the library's kernels (a kernel launched with
    # several grids, such as a GEMM split into a main launch and K-chunk
    # units, gets a row per grid)
    lines += ["", "Library kernels by launch grid (work-items in x):", "",
              "| kernel | grid | calls | average (us) | median (us) | total (ms) |", "|---|---|---|---|---|---|"]
    for (name, grid), v in sorted(shapes.items(), key=lambda kv: -sum(kv[1])):
        v = sorted(v)
        lines.append(f"| `{_short(name)[:70]}` | {grid} | {len(v)} | {sum(v) / len(v) / 1e3:.1f} | "
                     f"{v[len(v) // 2] / 1e3:.1f} | {sum(v) / 1e6:.2f} |")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter_per_dispatch(d: str, counter: str, pattern, reduce="sum") -> list:
    """Sum (or max) of `counter` over the instances of each matching dispatch."""
    per = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter or not pattern.search(r["Kernel_Name"]):
                continue
            k, v = (f, r["Dispatch_Id"]), float(r["Counter_Value"])
            per[k] = (per.get(k, 0.0) + v) if reduce == "sum" else max(per.get(k, v), v)
    return list(per.values())


def _mean(v):
    return sum(v) / len(v) if v else None


def _durations_ns(d: str, pattern) -> list:
    """End - start timestamp of each matching dispatch (one counter's rows)."""
    per = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if pattern.search(r["Kernel_Name"]):
                per[(f, r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
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
    # the other two kernels of the step, from the same runs
    others = {}
    for name, pat in (("activation pass (k_quantize)", QUANT_KERNEL), ("core GEMM (k_gemm, plain-store epilogue)", CORE_KERNEL),
                      ("one-kernel forward (k_fused: core and delta term in one K loop)", FUSED_KERNEL)):
        f = _mean(_counter_per_dispatch(run_fetch, "FETCH_SIZE", pat))
        w = _mean(_counter_per_dispatch(run_write, "WRITE_SIZE", pat))
        if f is not None and w is not None:
            others[name] = {"fetch_bytes": int(f * 1024 * f_scale), "write_bytes": int(w * 1024 * w_scale),
                            "traffic_bytes": int(f * 1024 * f_scale + w * 1024 * w_scale)}
    rec["other_kernels"] = others
    json.dump(rec, open(out, "w"), indent=1)
    print(json.dumps(rec, indent=1))


def summarize_mfma(run: str, out: str, cmd: str) -> None:
    lines = ["# MFMA counters: " + os.path.splitext(os.path.basename(out))[0], "",
             "Command (from the repository root on the GPU box):", "", "```", cmd, "```", "",
             "Per dispatch, averaged over the dispatches of each kernel (counter runs serialise dispatches).  "
             "MFMA flops = MOPS x 512.  GRBM_GUI_ACTIVE comes summed over the %d XCDs: active cycles = it / %d, "
             "clock = active cycles / dispatch duration.  MFMA utilisation = (SQ_VALU_MFMA_BUSY_CYCLES / %d SIMDs) / "
             "active cycles: the share of the kernel's cycles the average SIMD's matrix core is busy." % (XCDS, XCDS, SIMDS), "",
             "| kernel | dispatches | duration (us) | clock (GHz) | MFMA TFLOP F6F4 | MFMA TFLOP F8 | MFMA TFLOP BF16 | busy cycles / SIMD | active cycles | MFMA utilisation |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for name, pat in (("delta GEMM (k_gemm, token epilogue)", DELTA_KERNEL), ("core GEMM (k_gemm, plain store)", CORE_KERNEL),
                      ("activation pass (k_quantize)", QUANT_KERNEL), ("one-kernel forward (k_fused)", FUSED_KERNEL)):
        m4 = _counter_per_dispatch(run, "SQ_INSTS_VALU_MFMA_MOPS_F6F4", pat)
        m8 = _counter_per_dispatch(run, "SQ_INSTS_VALU_MFMA_MOPS_F8", pat)
        mb = _counter_per_dispatch(run, "SQ_INSTS_VALU_MFMA_MOPS_BF16", pat)
        busy = _counter_per_dispatch(run, "SQ_VALU_MFMA_BUSY_CYCLES", pat)
        act = _counter_per_dispatch(run, "GRBM_GUI_ACTIVE", pat, reduce="max")
        if not act:
            continue
        b, a = _mean(busy), _mean(act) / XCDS
        dur = _mean(_durations_ns(run, pat))
        lines.append(f"| {name} | {len(act)} | {dur / 1e3:.1f} | {a / dur:.2f} | {_mean(m4) * 512 / 1e12:.3f} | "
                     f"{_mean(m8) * 512 / 1e12:.3f} | {_mean(mb) * 512 / 1e12:.4f} | {b / SIMDS:.0f} | {a:.0f} | "
                     f"{100 * b / SIMDS / a:.1f} % |")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_issue(run: str, out: str, cmd: str, elements: int, probe: str = "", lds_run: str = "", lds_cmd: str = "") -> None:
    """Instruction issue per kernel: SQ_INSTS_{VALU,SALU,LDS} per dispatch
    and per wave, and the share of the average SIMD's cycles its VALU is
    issuing (a wave64 VALU instruction holds a 16-lane SIMD for 4 cycles)."""
    lines = ["# Instruction issue: " + os.path.splitext(os.path.basename(out))[0], "",
             "Command (from the repository root on the GPU box):", "", "```", cmd, "```", "",
             "Per dispatch, averaged over the dispatches of each kernel.  VALU issue share = SQ_INSTS_VALU x 4 cycles "
             "/ %d SIMDs / active cycles (GRBM_GUI_ACTIVE / %d XCDs); SQ_INSTS_VALU counts wave instructions, "
             "MFMAs included.  Lane-instructions per element = SQ_INSTS_VALU x 64 / %d activation elements "
             "(the activation pass only)." % (SIMDS, XCDS, elements), "",
             "| kernel | dispatches | duration (us) | clock (GHz) | waves | VALU / dispatch | VALU / wave | "
             "SALU / wave | LDS / wave | VALU issue share | VALU lane-instr / element |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for name, pat in (("activation pass (k_quantize)", QUANT_KERNEL), ("core GEMM (k_gemm, plain store)", CORE_KERNEL),
                      ("delta GEMM (k_gemm, token epilogue)", DELTA_KERNEL)):
        act = _counter_per_dispatch(run, "GRBM_GUI_ACTIVE", pat, reduce="max")
        if not act:
            continue
        waves = _mean(_counter_per_dispatch(run, "SQ_WAVES", pat))
        valu = _mean(_counter_per_dispatch(run, "SQ_INSTS_VALU", pat))
        salu = _mean(_counter_per_dispatch(run, "SQ_INSTS_SALU", pat))
        lds = _mean(_counter_per_dispatch(run, "SQ_INSTS_LDS", pat))
        a = _mean(act) / XCDS
        dur = _mean(_durations_ns(run, pat))
        per_el = f"{valu * 64 / elements:.1f}" if pat is QUANT_KERNEL else "-"
        lines.append(f"| {name} | {len(act)} | {dur / 1e3:.1f} | {a / dur:.2f} | {waves:.0f} | {valu:.4g} | "
                     f"{valu / waves:.0f} | {salu / waves:.0f} | {lds / waves:.0f} | "
                     f"{100 * valu * 4 / SIMDS / a:.1f} % | {per_el} |")
    if lds_run:
        lines += ["", "LDS bank conflicts (a second counter run):", "", "```", lds_cmd, "```", "",
                  "SQ_LDS_BANK_CONFLICT and SQ_INSTS_LDS come summed over every CU; conflict share = the conflict cycles "
                  "per CU (/ %d) over the active cycles." % CUS, "",
                  "| kernel | LDS instructions | bank-conflict cycles | per LDS instruction | conflict share |",
                  "|---|---|---|---|---|"]
        for name, pat in (("activation pass (k_quantize)", QUANT_KERNEL), ("core GEMM (k_gemm, plain store)", CORE_KERNEL),
                          ("delta GEMM (k_gemm, token epilogue)", DELTA_KERNEL)):
            act = _counter_per_dispatch(lds_run, "GRBM_GUI_ACTIVE", pat, reduce="max")
            if not act:
                continue
            n = _mean(_counter_per_dispatch(lds_run, "SQ_INSTS_LDS", pat))
            c = _mean(_counter_per_dispatch(lds_run, "SQ_LDS_BANK_CONFLICT", pat))
            a = _mean(act) / XCDS
            lines.append(f"| {name} | {n:.4g} | {c:.4g} | {c / n:.2f} | {100 * c / CUS / a:.1f} % |")
    if probe:
        lines += ["", "Plain streams on the same box (`python3 bench.py --stream-probe`):", "", "```", probe.strip(), "```"]
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


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
    if len(argv) >= 3 and argv[0] == "mfma":
        import argparse
        ap = argparse.ArgumentParser()
        ap.add_argument("run")
        ap.add_argument("out")
        ap.add_argument("--cmd", required=True)
        a = ap.parse_args(argv[1:])
        summarize_mfma(a.run, a.out, a.cmd)
        return
    if len(argv) >= 3 and argv[0] == "issue":
        import argparse
        ap = argparse.ArgumentParser()
        ap.add_argument("run")
        ap.add_argument("out")
        ap.add_argument("--cmd", required=True)
        ap.add_argument("--elements", type=int, required=True)
        ap.add_argument("--probe", default="", help="file holding a bench.py --stream-probe line")
        ap.add_argument("--lds", default="", help="a run with SQ_LDS_BANK_CONFLICT, SQ_INSTS_LDS, GRBM_GUI_ACTIVE")
        ap.add_argument("--lds-cmd", default="")
        a = ap.parse_args(argv[1:])
        probe = ""
        if a.probe:   # the JSON line only
            probe = "\n".join(l for l in open(a.probe).read().splitlines() if l.startswith("{"))
        summarize_issue(a.run, a.out, a.cmd, a.elements, probe, a.lds, a.lds_cmd)
        return
    raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
