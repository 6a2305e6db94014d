"""Benchmark of the delta-W4A4 linear layer on one MI355X.

One step = the whole hot path on one batch of synthetic activations already
resident in HBM: the activation pass (cube cores, deltas, MX codes, X L1)
followed by the forward GEMMs (core term, delta term, low-rank branch,
broadcast, token-order fp32 output), one dq_linear call, timed with HIP
events around the timed steps only.  Prints one JSON line.

value  = effective TOPS of the whole step, 2 N Ci Co / t_step (the dense
         layer's work; the method's own work differs, see 'work' below).
roofline = the dominant kernel, the delta GEMM (dq_delta_term: one launch of
         the FP4 x FP4 scaled-MFMA GEMM over the slots, with the low-rank
         branch, the core-term broadcast and the token-order stores in its
         epilogue): algorithmic FP4 flops per launch, 2 N Ci Co (one row per
         token: the pad slots of clipped cubes are executed but not counted;
         their share is reported as pad_slot_waste), / its average duration
         from HIP events on the launch stream (a second run of the steps,
         with events between the phases), against the dense FP4 peak;
         traffic from the committed rocprofv3 counter summary of the same
         kernel source, else null.  With one-token cubes the delta term is
         one FP8 x FP4 GEMM over the cubes and is rated against the FP8 peak.
fused_forward = the one-kernel form of the forward (dq_linear_forward_fused:
         core and delta partial sums in one K loop, no per-cube term in
         memory), timed beside the two kernels; dq_linear takes it on small
         layers (forward.form names the form the step runs).
cpu_baseline = the CPU oracle on a bounded sample of the same workload, its
         time extrapolated to the whole layer by the token count.

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
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: at least 20 and at least 0.25 s of them; the GPU clock ramps up "
                         "after the host-side weight preparation, over longer than 20 steps of a small layer take)")
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
    ap.add_argument("--orbit", action="store_true",
                    help="the rotated-basis W4A4 layer (RPBH + Lloyd-Max codebook) on the config's shape")
    ap.add_argument("--orbit-bits", type=int, default=4, choices=(2, 3, 4))
    ap.add_argument("--fp6", default="fp6_e2m3", choices=("fp6_e2m3", "fp6_e3m2"),
                    help="6-bit format of a text-token layer (--config kv_text_14b)")
    ap.add_argument("--stream-probe", action="store_true",
                    help="only measure plain streams of the activation pass's read/write mix and a device copy")
    ap.add_argument("--copy-only-mib", type=int, default=0,
                    help="only run 3 plain device-to-device copies of this size and exit (counter calibration)")
    return ap.parse_args()


def warm_up(step, warmup):
    """Untimed steps before the timed ones: `warmup` of them when given, else
    at least 20 and at least 0.25 s of them.  Returns the number run."""
    import time
    import torch

    n, t0 = 0, time.perf_counter()
    while (n < warmup) if warmup is not None else (n < 20 or time.perf_counter() - t0 < 0.25):
        step()
        n += 1
        if warmup is None and n % 10 == 0:
            torch.cuda.synchronize()            # the wall clock then follows the GPU
    torch.cuda.synchronize()
    return n


def time_steps(dq, weights, x, qa, y, stream, steps, warmup):
    """Mean ms per step over `steps` timed steps, each one dq_linear call
    (activation pass, core term, delta term), with HIP events on the launch
    stream around the steps only; then the mean ms of each phase from a
    second run of `steps` steps with events between the phases.  (Events
    between kernels leave gaps of several microseconds, so they stay out of
    the step time.)"""
    import numpy as np
    import torch

    ev = lambda: torch.cuda.Event(enable_timing=True)
    warmed = warm_up(lambda: dq.dq_linear(weights, x, qa, y, stream), warmup)
    start, end = ev(), ev()
    start.record(stream)
    for _ in range(steps):
        dq.dq_linear(weights, x, qa, y, stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / steps
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
    torch.cuda.synchronize()
    q_ms = float(np.mean([a.elapsed_time(b) for a, b, c, d in marks]))
    c_ms = float(np.mean([b.elapsed_time(c) for a, b, c, d in marks]))
    d_ms = float(np.mean([c.elapsed_time(d) for a, b, c, d in marks]))
    return ms_step, q_ms, c_ms, d_ms, warmed


def time_fused(dq, weights, qa, y, stream, steps):
    """Mean ms of dq_linear_forward_fused (the one-kernel forward: core and
    delta partial sums in one K loop) over `steps` calls on the state of one
    dq_quantize_act, HIP events on the launch stream; None where that form
    does not apply (it takes 4-token cubes with FP8 cores)."""
    import torch

    try:
        dq.dq_linear_forward_fused(weights, qa, y, stream)
    except dq.DQError:
        return None
    for _ in range(5):
        dq.dq_linear_forward_fused(weights, qa, y, stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        dq.dq_linear_forward_fused(weights, qa, y, stream)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


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
    # cubes of more than 64 tokens read X a second time (the partial-sum
    # pass): traffic beyond the algorithmic bytes, reported on its own
    xreread = sum(Ts * cfg.H * cfg.W for Ts, ts in segs if ts * h_ * w_ > 64) * Ci * xbytes
    return {
        "K": K, "S": S, "Nslot": Nslot, "N_tok": N,
        "dense": 2.0 * N * Ci * Co,
        "fp4": 2.0 * N * Ci * Co,            # delta term, one row per token (algorithmic)
        "fp4_slots": 2.0 * Nslot * Ci * Co,  # executed: one row per slot, pad slots of clipped cubes included
        "fp8": 2.0 * K * Ci * Co,            # core term, one row per cube (FP8, or FP4 cores)
        "bf16": 2.0 * N * r * (Ci + Co),     # low-rank branch
        # X once, delta codes and scales (not stored for one-token cubes: all
        # zero), core codes and scales (bf16 cores: their bf16 rows and the
        # FP8 codes, which the pass writes as well), U
        "quant_bytes": N * Ci * xbytes + (0 if S == 1 else N * Ci * (0.5 + 1 / 32))
                       + K * Ci * ((2 + 1) if core_bits == 16 else core_bits / 8) + K * Ci / 32 + 2 * N * r,
        "x_reread_bytes": xreread,
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
        print(json.dumps(shape_record(cfg, cube, *timing[:4], core_bits=args.core_bits)), flush=True)
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
                      {"ms": round(d_ms, 4), "fp4_tflops": round(wk["fp4"] / (d_ms * 1e-3) / 1e12, 1),
                       "pad_slot_waste": round(wk["fp4_slots"] / wk["fp4"] - 1, 4)},
        "core_overhead": core_overhead(wk, c_ms, d_ms, core_bits),
    }


def core_overhead(wk, c_ms, d_ms, core_bits=8):
    """The core term's cost next to the delta term's, the analogue of the
    pages' overhead figure for the core tokens' W4A8 GEMM (+3.2 % at cube size
    64, DeltaQuant page, 关键设计 4 and 亮点与洞察).  Measured: core-term time
    over delta-term time.  Rate model: the core GEMM has 1/S of the delta
    GEMM's rows and, for FP8 cores, runs at half the FP4 rate, so 2/S."""
    if wk["S"] == 1:
        return None
    rate = {8: 2.0, 4: 1.0, 16: 4.0}[core_bits]
    return {"measured_pct": round(100 * c_ms / d_ms, 2), "rate_model_pct": round(100 * rate * wk["K"] / wk["N_tok"], 2),
            "pages_pct_at_cube_64": 3.2}


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
        recs.append(shape_record(cfg, s, *time_steps(dq, weights, x, qa, y, stream, args.steps, args.warmup)[:4],
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


PEAK_FP6 = 10.1e15      # MI355X dense FP6 (the FP4 rate)


def bench_text(args, cfg, dq, torch):
    """The 6-bit layer on text tokens (the cross-attention K/V projections):
    one JSON line.  A step is dq_quantize_act6 (Q6(X), U) followed by
    dq_linear6_forward (the FP6 x FP6 GEMM with the low-rank branch), on the
    same stream; both timed with HIP events."""
    import numpy as np
    synth = synth_mod()
    fmt = args.fp6
    x = synth.make_text_activation(cfg.prompts, cfg.ctx, cfg.valid, cfg.Ci, cfg.x_seed, cfg.dtype,
                                   cfg.n_outliers).to("cuda:0")
    wt = synth.make_weight(cfg.Ci, cfg.Co, cfg.w_seed, cfg.dtype)
    l1, l2 = dq.dq_lowrank_factors(wt, cfg.rank, cfg.w_seed)
    weights = dq.dq_prepare_weights_w6(wt, l1, l2, fmt)
    act = dq.dq_act6_create(weights, cfg.N)
    y = torch.empty(cfg.N, cfg.Co, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    warmed = warm_up(lambda: dq.dq_linear6(weights, x, act, y, stream), args.warmup)
    start, end = ev(), ev()
    marks = []
    start.record(stream)
    for _ in range(args.steps):
        a, b, c = ev(), ev(), ev()
        a.record(stream)
        dq.dq_quantize_act6(weights, x, act, stream)
        b.record(stream)
        dq.dq_linear6_forward(weights, act, y, stream)
        c.record(stream)
        marks.append((a, b, c))
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    q_ms = float(np.mean([a.elapsed_time(b) for a, b, c in marks]))
    f_ms = float(np.mean([b.elapsed_time(c) for a, b, c in marks]))
    N, Ci, Co, r = cfg.N, cfg.Ci, cfg.Co, cfg.rank
    flops = 2.0 * N * Ci * Co
    xbytes = 2 if cfg.dtype == "bf16" else 4
    qbytes = N * Ci * xbytes + N * Ci * (0.75 + 1 / 32) + 2 * N * r
    out = {
        "metric": "effective TOPS of the 6-bit text-token layer (W6A6 + low rank)",
        "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": warmed, "ms_per_step": round(ms, 4), "higher_is_better": True, "dtype": fmt,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: X {N}x{Ci} ({cfg.prompts} contexts of {cfg.ctx} text tokens) {cfg.dtype} "
                               f"-> Y {N}x{Co} fp32, {fmt}, rank {r}", "tokens": N, "Ci": Ci, "Co": Co, "rank": r},
        "quantize": {"ms": round(q_ms, 4), "algorithmic_bytes": int(qbytes),
                     "GBps": round(qbytes / (q_ms * 1e-3) / 1e9, 1)},
        "roofline": {"kernel": "FP6 x FP6 GEMM (dq_linear6_forward: scaled MFMA, low-rank branch in the epilogue)",
                     "bound": "mfma", "achieved": round(flops / (f_ms * 1e-3) / 1e12, 2),
                     "peak": round(PEAK_FP6 / 1e12, 2), "unit": "TFLOP/s",
                     "frac": round(flops / (f_ms * 1e-3) / PEAK_FP6, 4), "ms": round(f_ms, 4),
                     "output_bytes": int(4 * N * Co), "weight_bytes": int(Co * Ci * (0.75 + 1 / 32))},
    }
    print(json.dumps(out), flush=True)


def bench_orbit(args, cfg, dq, torch):
    """The rotated-basis W4A4 layer (OrbitQuant notes: RPBH rotation,
    Lloyd-Max codebook) on a video layer's shape: one JSON line.  A step is
    dq_orbit_quantize_act (rotation, RMS, codes, decoded levels) followed by
    dq_orbit_forward (the bf16 GEMM over the decoded levels, scaled by the
    row scales), both timed with HIP events on the launch stream."""
    import numpy as np
    synth = synth_mod()
    x = synth.make_activation(cfg.T, cfg.H, cfg.W, cfg.Ci, seed=cfg.x_seeds[0], dtype=cfg.dtype,
                              n_outliers=cfg.n_outliers, device="cuda")
    wt = synth.config_weight(cfg)
    perm = np.random.default_rng(cfg.w_seed).permutation(cfg.Ci).astype(np.int32)
    o = dq.dq_orbit_prepare(wt, perm, args.orbit_bits, args.orbit_bits)
    act = dq.dq_orbit_act_create(o, cfg.N)
    y = torch.empty(cfg.N, cfg.Co, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    warmed = warm_up(lambda: dq.dq_orbit_linear(o, x, act, y, stream), args.warmup)
    start, end = ev(), ev()
    marks = []
    start.record(stream)
    for _ in range(args.steps):
        a, b, c = ev(), ev(), ev()
        a.record(stream)
        dq.dq_orbit_quantize_act(o, x, act, stream)
        b.record(stream)
        dq.dq_orbit_forward(o, act, y, stream)
        c.record(stream)
        marks.append((a, b, c))
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    q_ms = float(np.mean([a.elapsed_time(b) for a, b, c in marks]))
    f_ms = float(np.mean([b.elapsed_time(c) for a, b, c in marks]))
    N, Ci, Co = cfg.N, cfg.Ci, cfg.Co
    flops = 2.0 * N * Ci * Co
    qbytes = N * Ci * (2 if cfg.dtype == "bf16" else 4) + N * Ci * (0.5 + 2) + 4 * N
    print(json.dumps({
        "metric": "effective TOPS of the rotated-basis W4A4 layer (RPBH + Lloyd-Max codebook)",
        "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": warmed, "ms_per_step": round(ms, 4), "higher_is_better": True, "dtype": "bf16 (decoded levels)",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: X {N}x{Ci} {cfg.dtype} -> Y {N}x{Co} fp32, W{args.orbit_bits}A{args.orbit_bits} "
                               f"Lloyd-Max, blocks of 256", "tokens": N, "Ci": Ci, "Co": Co},
        "rotation": {"ms": round(q_ms, 4), "algorithmic_bytes": int(qbytes), "GBps": round(qbytes / (q_ms * 1e-3) / 1e9, 1)},
        "roofline": {"kernel": "bf16 GEMM over the decoded levels (dq_orbit_forward)", "bound": "mfma",
                     "achieved": round(flops / (f_ms * 1e-3) / 1e12, 2), "peak": round(PEAK_BF16 / 1e12, 2),
                     "unit": "TFLOP/s", "frac": round(flops / (f_ms * 1e-3) / PEAK_BF16, 4), "ms": round(f_ms, 4)},
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

    if args.stream_probe:
        stream_probe(args, torch)
        return
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
    if args.config in synth.TEXT_CONFIGS:
        bench_text(args, synth.TEXT_CONFIGS[args.config], dq, torch)
        return
    cfg = synth.CONFIGS[args.config]
    if args.orbit:
        bench_orbit(args, cfg, dq, torch)
        return
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
    ms_step, q_ms, c_ms, d_ms, warmed = time_steps(dq, weights, x, qa, y, stream, args.steps, args.warmup)
    fused_ms = time_fused(dq, weights, qa, y, stream, args.steps)
    form = dq.dq_forward_form(weights, qa)          # the form dq_linear's forward takes for this layer
    ctype = "bf16" if args.core_bits == 16 else f"fp{args.core_bits}"      # the core GEMM's input type
    f_ms = fused_ms if form == "one kernel" and fused_ms is not None else c_ms + d_ms
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
    # the dominant kernel: the delta GEMM (FP4 x FP4) on 2 N Ci Co; with
    # one-token cubes it is the FP8 x FP4 GEMM over the cubes (FP4 x FP4 for
    # FP4 cores), on 2 K Ci Co
    rl_ms = d_ms
    if S == 1:
        rl_flops, rl_peak = f_fp8, {8: PEAK_FP8, 4: PEAK_FP4, 16: PEAK_FP8}[args.core_bits]
        rl_kernel = ("GEMM over the one-token cubes (dq_delta_term: FP8 x FP4 scaled MFMA, Q8(x) Q4(R); "
                     "low-rank branch and token-order stores in the epilogue)")
    elif form == "one kernel":
        # the one-kernel forward: both contractions, the FP8 x FP4 flops
        # counted at the FP4 peak's rate (PEAK_FP4 / PEAK_FP8 each), so frac
        # is the time both would take at their peaks over the measured time
        rl_flops, rl_peak, rl_ms = f_fp4 + f_fp8 * PEAK_FP4 / PEAK_FP8, PEAK_FP4, fused_ms
        rl_kernel = ("one-kernel forward (dq_linear_forward_fused: FP4 x FP4 delta and FP8 x FP4 core MFMAs in one "
                     "K loop, FP8 flops counted at the FP4 rate; low-rank branch, core term and token-order stores "
                     "in the epilogue)")
    else:
        rl_flops, rl_peak = f_fp4, PEAK_FP4
        rl_kernel = ("delta GEMM (dq_delta_term: FP4 x FP4 scaled MFMA over the slots; low-rank branch, "
                     "core-term broadcast and token-order stores in the epilogue)")
    achieved = rl_flops / (rl_ms * 1e-3)
    traffic = committed_traffic(args.config, cube) if form == "two kernels" or S == 1 else None

    cpu = sanity = None
    if not args.no_cpu_baseline:
        cpu, sanity = cpu_baseline(cfg, cube, x, y, weights, dq, args.cpu_tokens)

    out = {
        "metric": "effective TOPS of fused delta-W4A4 linear + % of MI355X FP4 MFMA peak",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmed,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4" if args.core_bits == 4 else ("mxfp4+bf16" if args.core_bits == 16 else "mxfp4+mxfp8"),
        "precision": ("deltas and R in MX-FP4 (FP4 x FP4 scaled MFMA: each 64-term block exact, rounded once into "
                      "fp32); cores in " + {8: "MX-FP8 (FP8 x FP4 scaled MFMA keeps about 13 bits per block)",
                                            4: "MX-FP4", 16: "bf16 (bf16 MFMA, fp32 accumulation)"}[args.core_bits]
                      + "; low-rank branch in bf16 with fp32 accumulation; fp32 output"),
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: X {N}x{Ci} ({T}x{H}x{W} tokens) {cfg.dtype} -> Y {N}x{Co} fp32, "
                        f"cube {t_}x{h_}x{w_}, rank {r}",
            "tokens": N, "Ci": Ci, "Co": Co, "cube": list(cube), "rank": r, "cubes": K,
            "core_group": args.core_group, "core_bits": args.core_bits,
        },
        "pct_fp4_peak_step": round(100 * dense_flops / (ms_step * 1e-3) / PEAK_FP4, 2),
        "forward": {
            "form": form,
            "ms": round(f_ms, 4),
            "effective_tops": round(dense_flops / (f_ms * 1e-3) / 1e12, 2),
            "pct_fp4_peak": round(100 * dense_flops / (f_ms * 1e-3) / PEAK_FP4, 2),
        },
        "quantize": {
            "ms": round(q_ms, 4),
            "algorithmic_bytes": int(quant_bytes),
            "x_reread_bytes": int(wk["x_reread_bytes"]),
            "GBps": round(quant_bytes / (q_ms * 1e-3) / 1e9, 1),
            "pct_hbm": round(100 * quant_bytes / (q_ms * 1e-3) / PEAK_HBM, 2),
            "copy_GBps": round(copy_gbps, 1),
            "pct_copy": round(100 * quant_bytes / (q_ms * 1e-3) / 1e9 / copy_gbps, 2),
        },
        "core_overhead": core_overhead(wk, c_ms, d_ms, args.core_bits),
        # the one-kernel form of the forward (dq_linear_forward_fused), which
        # the step uses on small layers (forward.form)
        "fused_forward": None if fused_ms is None else {
            "ms": round(fused_ms, 4),
            "vs_two_kernels": round(fused_ms / (c_ms + d_ms), 4),
            "effective_tops": round(dense_flops / (fused_ms * 1e-3) / 1e12, 2),
            "hbm_saved_bytes": int(2 * 4 * K * Co),
        },
        "core_term": {
            "ms": round(c_ms, 4),
            f"{ctype}_tflops": round(f_fp8 / (c_ms * 1e-3) / 1e12, 2),
            f"pct_{ctype}_peak": round(100 * f_fp8 / (c_ms * 1e-3) / {8: PEAK_FP8, 4: PEAK_FP4, 16: PEAK_BF16}[args.core_bits], 2),
        },
        "roofline": {
            "kernel": rl_kernel,
            "bound": "mfma",
            "achieved": round(achieved / 1e12, 2),
            "peak": round(rl_peak / 1e12, 2),
            "unit": "TFLOP/s",
            "frac": round(achieved / rl_peak, 4),
            "traffic": traffic,
            "ms": round(rl_ms, 4),
            "work": {"fp4_flops": f_fp4, "fp4_flops_executed": wk["fp4_slots"], "fp8_flops": f_fp8,
                     "bf16_flops": f_bf16},
            "pad_slot_waste": round(wk["fp4_slots"] / f_fp4 - 1, 4),
        },
        "cpu_baseline": cpu,
        "sanity_error": sanity,
    }
    print(json.dumps(out), flush=True)


def stream_probe(args, torch):
    """The attainable HBM rate for the activation pass's traffic mix: a
    plain elementwise kernel that reads the whole of a layer's X and writes
    half of its bytes (the pass reads X once and writes its codes, scales
    and U, about 0.4 of X's bytes), next to a plain device copy.  One JSON
    line."""
    from w4a4_quantized_linear_cube_amd import synth
    cfg = synth.CONFIGS[args.config]
    x = synth.make_activation(cfg.T, cfg.H, cfg.W, cfg.Ci, seed=cfg.x_seeds[0], dtype=cfg.dtype,
                              n_outliers=cfg.n_outliers, device="cuda")
    xi = x.view(torch.int32)                       # 2-byte or 4-byte elements alike
    half = xi.shape[1] // 2
    a, b = xi[:, :half], xi[:, half:2 * half]
    out = torch.empty(xi.shape[0], half, dtype=torch.int32, device=x.device)
    dst = torch.empty_like(x)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def rate(fn, nbytes, reps=20):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        s0, s1 = ev(), ev()
        s0.record()
        for _ in range(reps):
            fn()
        s1.record()
        torch.cuda.synchronize()
        return nbytes * reps / (s0.elapsed_time(s1) * 1e-3) / 1e9

    xb = x.numel() * x.element_size()
    mix = rate(lambda: torch.bitwise_xor(a, b, out=out), xb + out.numel() * 4)
    copy = rate(lambda: dst.copy_(x), 2 * xb)
    print(json.dumps({"probe": "stream", "config": cfg.name, "read_bytes": xb, "write_bytes": out.numel() * 4,
                      "mix_GBps": round(mix, 1), "copy_GBps": round(copy, 1),
                      "mix_pct_hbm": round(100 * mix / (PEAK_HBM / 1e9), 2)}), flush=True)


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


def cpu_baseline(cfg, cube, x, y, weights, dq, n_tokens):
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
    base = {
        "value": round(2.0 * n * cfg.Ci * cfg.Co / dt / 1e12, 6),
        "unit": "TOPS",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{len(ids)} whole cubes ({n} of {cfg.N} tokens) of the same layer: activation pass + forward, "
                  f"{dt:.2f} s wall; the whole layer extrapolated by the token count",
        "extrapolated": True,
        "full_layer_s": round(dt * cfg.N / n, 1),
    }
    # Sanity check (untimed): the layer output's error against the exact
    # X W (fp64) on 256 of the sampled tokens, for delta W4A4 (the GPU's y of
    # the timed steps) and for direct W4A4 of X (the oracle: the same R,
    # rank, low-rank branch and MX rule, X quantized per token, no cubes).
    sel = np.sort(rng.choice(n, size=min(256, n), replace=False))
    tk = np.asarray(q["tokens"])[sel]
    ex = layer.exact_output(xf[tk], wf)
    yg = y.index_select(0, torch.from_numpy(tk).to(y.device)).cpu().numpy()
    yd = layer.direct_output(xf[tk], q["U"][sel], l2, rc, rs)
    sanity = {"tokens": int(len(tk)), "rel_err_delta_w4a4": round(layer.rel_fro(yg, ex), 5),
              "rel_err_direct_w4a4": round(layer.rel_fro(yd, ex), 5),
              "against": "exact X W in fp64; delta: the GPU output, direct: the oracle with X quantized per token"}
    return base, sanity


if __name__ == "__main__":
    main()
