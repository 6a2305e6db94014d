"""Benchmark of the delta-W4A4 linear layer on one MI355X.

One step = the whole hot path on one batch of synthetic activations already
resident in HBM: the activation pass (cube cores, deltas, MX codes, X L1)
followed by the forward GEMMs (core term, delta term, low-rank branch,
broadcast, token-order fp32 output).  Prints one JSON line.

value  = effective TOPS of the whole step, 2 N Ci Co / t_step (the dense
         layer's work; the method's own work differs, see 'work' below).
roofline = the dominant kernel, the delta GEMM (dq_delta_term: one launch of
         the FP4 x FP4 scaled-MFMA GEMM over the slots, with the low-rank
         branch, the core-term broadcast and the token-order stores in its
         epilogue): algorithmic FP4 flops per launch, 2 N_slot Ci Co, / its
         average duration from HIP events on the launch stream, against the
         dense FP4 peak; traffic from the committed rocprofv3 counter summary
         of the same kernel source, else null.
cpu_baseline = the CPU oracle on a bounded sample of the same workload.

--sweep instead prints one JSON line per cube shape of the config's list
(e.g. --config ffn_down_720p --sweep: 1x1x1, 1x2x2, 2x2x2, 1x4x4 and one
global cube) with the step time, effective TOPS and the three phases.
--schedule prints the same for the timestep-aware cube sizes (4x1x4, then
4x2x8), and one line for a whole denoising run of the layer that switches
between them.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published dense peaks
PEAK_FP4 = 10.1e15
PEAK_FP8 = 5.0e15
PEAK_BF16 = 2.5e15
PEAK_HBM = 8.0e12


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps first (20: the GPU clock ramps up after the host-side weight preparation)")
    ap.add_argument("--config", default="ffn_up_720p")
    ap.add_argument("--cube", default=None, help="t,h,w (default: the config's first cube)")
    ap.add_argument("--x-seed", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=24576, help="tokens in the oracle's timed sample (about 10 s of host work)")
    ap.add_argument("--sweep", action="store_true", help="one JSON line per cube shape of the config")
    ap.add_argument("--schedule", action="store_true",
                    help="the timestep-aware cube schedule (4x1x4 early, 4x2x8 after) on the config's layer")
    ap.add_argument("--denoise-steps", type=int, default=10, help="denoising steps of one --schedule run")
    ap.add_argument("--core-group", type=int, default=32, choices=(32, 64),
                    help="channels per FP8 exponent of the cores (64: the pages' group size)")
    ap.add_argument("--core-bits", type=int, default=8, choices=(8, 4, 16),
                    help="MX-FP8 cores (the pages' choice), MX-FP4 or bf16 cores (the 4- and 16-bit points of their ablation)")
    ap.add_argument("--copy-only-mib", type=int, default=0,
                    help="only run 3 plain device-to-device copies of this size and exit (counter calibration)")
    return ap.parse_args()


def time_steps(dq, weights, x, qa, y, stream, steps, warmup):
    """Mean ms per step and per phase (activation pass, core term, delta
    term) over `steps` timed steps, HIP events on the launch stream."""
    import numpy as np
    import torch

    ev = lambda: torch.cuda.Event(enable_timing=True)
    for _ in range(warmup):
        dq.dq_linear(weights, x, qa, y, stream)
    torch.cuda.synchronize()
    start, end = ev(), ev()
    start.record(stream)
    marks = []
    for _ in range(steps):
        a, b, c, d = ev(), ev(), ev(), ev()
        a.record(stream)
        dq.dq_quantize_act(weights, x, qa, stream)
        b.record(stream)
        dq.dq_core_term(weights, qa, stream)
        c.record(stream)
        dq.dq_delta_term(weights, qa, y, stream)
        d.record(stream)
        marks.append((a, b, c, d))
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / steps
    q_ms = float(np.mean([a.elapsed_time(b) for a, b, c, d in marks]))
    c_ms = float(np.mean([b.elapsed_time(c) for a, b, c, d in marks]))
    d_ms = float(np.mean([c.elapsed_time(d) for a, b, c, d in marks]))
    return ms_step, q_ms, c_ms, d_ms


def work(cfg, cube, core_bits=8):
    """Sizes of the method's work for a cube shape: cubes, slots, flops of
    each GEMM, the activation pass's algorithmic bytes."""
    t_, h_, w_ = cube
    Hc, Wc = -(-cfg.H // h_), -(-cfg.W // w_)
    S = t_ * h_ * w_
    N, Ci, Co, r = cfg.N, cfg.Ci, cfg.Co, cfg.rank
    xbytes = 2 if cfg.dtype == "bf16" else 4
    # frame segments: the whole frame groups, then the last T % t frames as
    # cubes of T % t frames (no pad slots for the missing frames)
    T0 = cfg.T - cfg.T % t_
    segs = [(T0, t_)] + ([(cfg.T - T0, cfg.T - T0)] if T0 < cfg.T else [])
    K = sum(-(-Ts // ts) * Hc * Wc for Ts, ts in segs)
    Nslot = sum(-(-Ts // ts) * Hc * Wc * ts * h_ * w_ for Ts, ts in segs)
    # X once (twice in a segment of cubes of more than 64 tokens)
    xreads = sum(Ts * cfg.H * cfg.W * (2 if ts * h_ * w_ > 64 else 1) for Ts, ts in segs)
    return {
        "K": K, "S": S, "Nslot": Nslot,
        "dense": 2.0 * N * Ci * Co,
        "fp4": 2.0 * Nslot * Ci * Co,        # delta term, one row per slot (pad slots of clipped cubes included)
        "fp8": 2.0 * K * Ci * Co,            # core term, one row per cube (FP8, or FP4 cores)
        "bf16": 2.0 * N * r * (Ci + Co),     # low-rank branch
        # X, delta codes and scales (not stored for one-token cubes: all
        # zero), core codes and scales (bf16 cores: their bf16 rows and the
        # FP8 codes, which the pass writes as well), U
        "quant_bytes": xreads * Ci * xbytes + (0 if S == 1 else N * Ci * (0.5 + 1 / 32))
                       + K * Ci * ((2 + 1) if core_bits == 16 else core_bits / 8) + K * Ci / 32 + 2 * N * r,
    }


def sweep(args, cfg, dq, torch):
    """One JSON line per cube shape of the config (same weights, same X)."""
    wt = synth_mod().config_weight(cfg)
    weights = dq.dq_prepare_weights(wt, cfg.rank, seed=cfg.w_seed, device=0)
    x = synth_mod().make_activation(cfg.T, cfg.H, cfg.W, cfg.Ci, seed=cfg.x_seeds[0], dtype=cfg.dtype,
                                    n_outliers=cfg.n_outliers, device="cuda")
    y = torch.empty(cfg.N, cfg.Co, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    for cube in cfg.cubes:
        qa = dq.dq_qact_create(weights, (cfg.T, cfg.H, cfg.W) + tuple(cube), core_group=args.core_group, core_bits=args.core_bits)
        timing = time_steps(dq, weights, x, qa, y, stream, args.steps, args.warmup)
        print(json.dumps(shape_record(cfg, cube, *timing, core_bits=args.core_bits)), flush=True)
        torch.cuda.synchronize()
        del qa                      # frees the cube shape's buffers


def shape_record(cfg, cube, ms, q_ms, c_ms, d_ms, core_bits=8):
    """One cube shape's step time, split by phase, with its rates."""
    wk = work(cfg, cube, core_bits)
    one = wk["S"] == 1          # one-token cubes: the delta term is one GEMM over the cubes (FP8 or FP4 cores)
    ck = ("bf16" if core_bits == 16 else f"fp{core_bits}") + "_tflops"
    return {
        "config": cfg.name, "cube": list(cube), "cubes": wk["K"], "slots": wk["Nslot"],
        "ms_per_step": round(ms, 4), "effective_tops": round(wk["dense"] / (ms * 1e-3) / 1e12, 2),
        "quantize": {"ms": round(q_ms, 4), "GBps": round(wk["quant_bytes"] / (q_ms * 1e-3) / 1e9, 1)},
        "core_term": {"ms": round(c_ms, 4)} if one else
                     {"ms": round(c_ms, 4), ck: round(wk["fp8"] / (c_ms * 1e-3) / 1e12, 1)},
        "delta_term": {"ms": round(d_ms, 4), ck: round(wk["fp8"] / (d_ms * 1e-3) / 1e12, 1)} if one else
                      {"ms": round(d_ms, 4), "fp4_tflops": round(wk["fp4"] / (d_ms * 1e-3) / 1e12, 1)},
    }


# Timestep-aware cube sizes (DeltaQuant notes, 损失函数/训练策略): 16-token
# cubes (t4 h1 w4) for the first 25-30 % of the denoising steps (high noise,
# the steps that matter most for quality), 64-token cubes (t4 h2 w8) for the
# rest.  30 % here.
SCHEDULE_SHAPES = ((4, 1, 4), (4, 2, 8))
SCHEDULE_EARLY = 0.3


def schedule(args, cfg, dq, torch):
    """The cube schedule on one layer: a JSON line per cube shape, then one
    for a whole denoising run of the layer (the shape switches after the
    early steps; both handles stay allocated, so switching costs nothing)."""
    wt = synth_mod().config_weight(cfg)
    weights = dq.dq_prepare_weights(wt, cfg.rank, seed=cfg.w_seed, device=0)
    x = synth_mod().make_activation(cfg.T, cfg.H, cfg.W, cfg.Ci, seed=cfg.x_seeds[0], dtype=cfg.dtype,
                                    n_outliers=cfg.n_outliers, device="cuda")
    y = torch.empty(cfg.N, cfg.Co, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    qas = [dq.dq_qact_create(weights, (cfg.T, cfg.H, cfg.W) + s, core_group=args.core_group, core_bits=args.core_bits) for s in SCHEDULE_SHAPES]
    recs = []
    for s, qa in zip(SCHEDULE_SHAPES, qas):
        recs.append(shape_record(cfg, s, *time_steps(dq, weights, x, qa, y, stream, args.steps, args.warmup),
                                 core_bits=args.core_bits))
        print(json.dumps(recs[-1]), flush=True)
    n = args.denoise_steps
    n_early = max(1, min(n, round(SCHEDULE_EARLY * n)))
    plan = [qas[0]] * n_early + [qas[1]] * (n - n_early)
    for qa in plan:                 # warm-up: one run
        dq.dq_linear(weights, x, qa, y, stream)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    runs = max(1, args.steps // n)
    start.record(stream)
    for _ in range(runs):
        for qa in plan:
            dq.dq_linear(weights, x, qa, y, stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms_call = start.elapsed_time(end) / (runs * n)
    dense = work(cfg, SCHEDULE_SHAPES[0])["dense"]
    print(json.dumps({
        "config": cfg.name, "schedule": [["x".join(map(str, SCHEDULE_SHAPES[0])), n_early],
                                         ["x".join(map(str, SCHEDULE_SHAPES[1])), n - n_early]],
        "denoise_steps": n, "runs": runs, "ms_per_layer_call": round(ms_call, 4),
        "effective_tops": round(dense / (ms_call * 1e-3) / 1e12, 2),
        "predicted_ms_per_layer_call": round((n_early * recs[0]["ms_per_step"] + (n - n_early) * recs[1]["ms_per_step"]) / n, 4),
    }), flush=True)


def synth_mod():
    from w4a4_quantized_linear_cube_amd import synth
    return synth


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer shards by whole cubes "
              "along tokens with no communication, so per-GPU throughput is the one-GPU number.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_only_mib:
        nbytes = args.copy_only_mib << 20
        src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copies: 3 x {nbytes} bytes read and written", file=sys.stderr, flush=True)
        return

    from w4a4_quantized_linear_cube_amd import dq, synth

    if not os.path.exists(dq.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    dq.load()
    cfg = synth.CONFIGS[args.config]
    if args.sweep:
        sweep(args, cfg, dq, torch)
        return
    if args.schedule:
        schedule(args, cfg, dq, torch)
        return
    cube = tuple(int(v) for v in args.cube.split(",")) if args.cube else cfg.cubes[0]
    xseed = cfg.x_seeds[0] if args.x_seed is None else args.x_seed
    T, H, W, Ci, Co, r = cfg.T, cfg.H, cfg.W, cfg.Ci, cfg.Co, cfg.rank
    N = cfg.N
    dev = torch.device("cuda:0")
    print(f"[bench] {cfg.name} N={N} Ci={Ci} Co={Co} cube={cube} r={r}: preparing", file=sys.stderr, flush=True)

    wt = synth.config_weight(cfg)
    weights = dq.dq_prepare_weights(wt, r, seed=cfg.w_seed, device=0)
    qa = dq.dq_qact_create(weights, (T, H, W) + cube, core_group=args.core_group, core_bits=args.core_bits)
    x = synth.make_activation(T, H, W, Ci, seed=xseed, dtype=cfg.dtype, n_outliers=cfg.n_outliers, device="cuda")
    y = torch.empty(N, Co, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    # derived sizes of the method's work
    t_, h_, w_ = cube
    wk = work(cfg, cube, args.core_bits)
    K, S = wk["K"], wk["S"]
    dense_flops, f_fp4, f_fp8, f_bf16, quant_bytes = wk["dense"], wk["fp4"], wk["fp8"], wk["bf16"], wk["quant_bytes"]

    # timed steps (activation pass, core term, delta term: dq_linear's work);
    # per-phase events on the launch stream
    ms_step, q_ms, c_ms, d_ms = time_steps(dq, weights, x, qa, y, stream, args.steps, args.warmup)
    ctype = "bf16" if args.core_bits == 16 else f"fp{args.core_bits}"      # the core GEMM's input type
    f_ms = c_ms + d_ms
    ev = lambda: torch.cuda.Event(enable_timing=True)

    # device-to-device copy rate (the practical ceiling of the activation pass)
    cbytes = 1 << 30
    csrc = torch.empty(cbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    c0, c1 = ev(), ev()
    c0.record(stream)
    for _ in range(5):
        cdst.copy_(csrc)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * cbytes * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del csrc, cdst

    value = dense_flops / (ms_step * 1e-3) / 1e12
    achieved = f_fp4 / (d_ms * 1e-3)
    traffic = committed_traffic(args.config, cube)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, cube, x, weights, dq, args.cpu_tokens)

    out = {
        "metric": "effective TOPS of fused delta-W4A4 linear + % of MI355X FP4 MFMA peak",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"mxfp4 (deltas, R) + {'bf16' if args.core_bits == 16 else 'mxfp%d' % args.core_bits} (cores) + bf16 (low rank), fp32 accumulate",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: X {N}x{Ci} ({T}x{H}x{W} tokens) {cfg.dtype} -> Y {N}x{Co} fp32, "
                        f"cube {t_}x{h_}x{w_}, rank {r}",
            "tokens": N, "Ci": Ci, "Co": Co, "cube": list(cube), "rank": r, "cubes": K,
            "core_group": args.core_group, "core_bits": args.core_bits,
        },
        "pct_fp4_peak_step": round(100 * dense_flops / (ms_step * 1e-3) / PEAK_FP4, 2),
        "forward": {
            "ms": round(f_ms, 4),
            "effective_tops": round(dense_flops / (f_ms * 1e-3) / 1e12, 2),
            "pct_fp4_peak": round(100 * dense_flops / (f_ms * 1e-3) / PEAK_FP4, 2),
        },
        "quantize": {
            "ms": round(q_ms, 4),
            "algorithmic_bytes": int(quant_bytes),
            "GBps": round(quant_bytes / (q_ms * 1e-3) / 1e9, 1),
            "pct_hbm": round(100 * quant_bytes / (q_ms * 1e-3) / PEAK_HBM, 2),
            "copy_GBps": round(copy_gbps, 1),
            "pct_copy": round(100 * quant_bytes / (q_ms * 1e-3) / 1e9 / copy_gbps, 2),
        },
        "core_term": {
            "ms": round(c_ms, 4),
            f"{ctype}_tflops": round(f_fp8 / (c_ms * 1e-3) / 1e12, 2),
            f"pct_{ctype}_peak": round(100 * f_fp8 / (c_ms * 1e-3) / {8: PEAK_FP8, 4: PEAK_FP4, 16: PEAK_BF16}[args.core_bits], 2),
        },
        "roofline": {
            "kernel": "delta GEMM (dq_delta_term: FP4 x FP4 scaled MFMA over the slots; low-rank branch, "
                      "core-term broadcast and token-order stores in the epilogue)",
            "bound": "mfma",
            "achieved": round(achieved / 1e12, 2),
            "peak": round(PEAK_FP4 / 1e12, 2),
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP4, 4),
            "traffic": traffic,
            "ms": round(d_ms, 4),
            "work": {"fp4_flops": f_fp4, "fp8_flops": f_fp8, "bf16_flops": f_bf16},
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def committed_traffic(config, cube):
    """HBM bytes per launch of the delta GEMM from the committed counter
    summary (profiles/delta_gemm_<config>_traffic.json: FETCH_SIZE and
    WRITE_SIZE per dispatch, each scaled by the same counter's reading for a
    plain copy of known size), if it was taken on this workload and on the
    current kernel source; else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"delta_gemm_{config}_traffic.json")
    src = os.path.join(ROOT, "w4a4_quantized_linear_cube_amd", "csrc", "gemm.hip")
    try:
        rec = json.load(open(path))
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("gemm_hip_sha256") != digest or list(rec.get("cube", [])) != list(cube):
        return None
    return rec.get("traffic_bytes")


def cpu_baseline(cfg, cube, x, weights, dq, n_tokens):
    """The oracle, as it stands, on a bounded sample: whole cubes covering
    about n_tokens tokens, quantized and pushed through the layer on the host
    (weights prepared beforehand and not timed, as on the GPU)."""
    import numpy as np

    from oracle import cubes, layer, lowrank
    from w4a4_quantized_linear_cube_amd import synth

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    e = dq.dq_weights_export(weights)
    l1, l2 = e["l1"], e["l2"]          # the host-SVD factors: inputs, like W
    wf = synth.to_f32_numpy(synth.config_weight(cfg))
    rc, rs = lowrank.quantize_residual(lowrank.residual(wf, l1, l2))   # weight preparation, not timed
    g = cubes.Geometry(cfg.T, cfg.H, cfg.W, *cube)
    rng = np.random.default_rng(0)
    n_cubes = max(1, n_tokens // g.S)
    ids = np.sort(rng.choice(g.K, size=min(n_cubes, g.K), replace=False))
    tbl, _ = cubes.cube_tokens(g, ids)
    toks = np.sort(tbl[tbl >= 0])
    if len(toks) > 4 * n_tokens:
        toks = toks[:n_tokens]
    # activation rows the sample touches, from the device copy of the input
    import torch
    xf = np.zeros((cfg.N, cfg.Ci), dtype=np.float32)
    need = torch.from_numpy(np.unique(tbl[tbl >= 0])).to(x.device)
    xf[need.cpu().numpy()] = x.index_select(0, need).float().cpu().numpy()
    t0 = time.perf_counter()
    q = layer.quantize_activation(xf, g, l1, cube_ids=ids, tokens=toks)
    yo = layer.forward(q, g, rc, rs, l2)
    dt = time.perf_counter() - t0
    n = len(q["tokens"])
    return {
        "value": round(2.0 * n * cfg.Ci * cfg.Co / dt / 1e12, 6),
        "unit": "TOPS",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{len(ids)} whole cubes ({n} tokens) of the same layer: activation pass + forward, "
                  f"{dt:.2f} s wall",
    }


if __name__ == "__main__":
    main()
