"""Helpers of the GPU parity tests: the comparison bars against the oracle.

Codes and scale codes are compared bit for bit; U within one bf16 ulp plus
the fp32 summation bound; y within 2e-3 relative Frobenius error, every
element inside an accumulation bound derived from the instruction
precisions, and every row within ROW_TOL (a misplaced or wrong row is off by
O(1); single rows whose terms cancel can exceed 2e-3, see _check_y).
"""
import sys

import numpy as np
import torch

from oracle import cubes, layer, lowrank, mx
from w4a4_quantized_linear_cube_amd import synth

DEV = "cuda:0"
TOL = 2e-3
ROW_TOL = 1e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _random_factors(Ci, Co, r, seed):
    """Seeded bf16 factors of realistic magnitude (not an SVD)."""
    if r == 0:
        return np.zeros((Ci, 0), np.uint16), np.zeros((0, Co), np.uint16)
    g = torch.Generator().manual_seed(seed)
    l1 = (torch.randn(Ci, r, generator=g) * 0.05).to(torch.bfloat16)
    l2 = (torch.randn(r, Co, generator=g) * 0.05).to(torch.bfloat16)
    return (l1.view(torch.int16).numpy().view(np.uint16).copy(), l2.view(torch.int16).numpy().view(np.uint16).copy())


def _ulp_bf16(v):
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def _check_u(got_bits, want_bits, x_rows, l1_bits):
    """U = bf16(bf16(x) L1) with fp32 accumulation on the GPU vs fp64 in the
    oracle: they may differ by one bf16 ulp of rounding plus the fp32
    summation error bound (Ci - 1) 2^-24 sum_c |x_c L1_c| (any order)."""
    g = mx.bf16_bits_to_f64(got_bits)
    w = mx.bf16_bits_to_f64(want_bits)
    xb = np.abs(mx.bf16_bits_to_f64(mx.f32_to_bf16_bits(x_rows)))
    absdot = xb @ np.abs(mx.bf16_bits_to_f64(l1_bits))
    bound = _ulp_bf16(np.maximum(np.abs(g), np.abs(w))) + (x_rows.shape[1] - 1) * 2.0 ** -24 * absdot
    bad = np.argwhere(np.abs(g - w) > bound)
    assert len(bad) == 0, f"U outside the fp32-accumulation bound at {bad[:5]}"


# Per-instruction accuracy of the gfx950 scaled MFMA, measured on random
# full-lane data against exact sums: FP4 x FP4 returns the exact 64-term sum
# rounded once (<= 0.5 ulp; two roundings with a nonzero accumulator), while
# FP8 x FP4 keeps about 13 bits internally (worst 2^-12.6 of sum|products|
# per instruction on random codes, 2^-10.5 with mostly subnormal FP8).
MFMA_FP8_REL = 2.0 ** -9


def _abs_bound(q, g, rc, rs, l2_bits, x_rows, l1_bits):
    """Elementwise bound on |y_gpu - y_oracle| from the arithmetic: the delta
    dot product is Ci/64 MFMA blocks of exact sums each rounded (twice) into an
    fp32 accumulator; the core dot product the same plus MFMA_FP8_REL per
    block; the low-rank dot product r/16 bf16 blocks; plus the low-rank term's
    share of the U difference allowed by _check_u.  The final rounding of y is
    added by the caller."""
    Ci = rc.shape[1] * 2
    r = l2_bits.shape[0]
    rdq = np.abs(mx.mx_dequantize(mx.unpack_fp4(rc), rs, "fp4")).T
    core_abs = np.abs(layer.core_values(q))
    delta_abs = np.abs(mx.mx_dequantize(mx.unpack_fp4(q["delta_codes"]), q["delta_scales"], "fp4"))
    rows = q["row_of_cube"][cubes.cube_of_token(g, q["tokens"])]
    blocks = Ci // 64 + 4
    bound = (blocks * 2.0 ** -23) * (delta_abs @ rdq) + (MFMA_FP8_REL + blocks * 2.0 ** -23) * (core_abs @ rdq)[rows]
    # subnormal partial results: an MFMA block result or accumulator step that
    # falls below 2^-126 may be flushed, losing at most 2^-126 each
    bound = bound + (2 * blocks + r // 16 + 4) * 2.0 ** -126
    if r:
        u = np.abs(mx.bf16_bits_to_f64(q["U"]))
        l2a = np.abs(mx.bf16_bits_to_f64(l2_bits))
        xb = np.abs(mx.bf16_bits_to_f64(mx.f32_to_bf16_bits(x_rows)))
        ub = 2 * _ulp_bf16(u) + (Ci - 1) * 2.0 ** -24 * (xb @ np.abs(mx.bf16_bits_to_f64(l1_bits)))
        bound = bound + ((r // 16 + 4) * 2.0 ** -23) * ((u + ub) @ l2a) + ub @ l2a
    return bound


def _check_y(y, yo, bound=None):
    err = layer.rel_fro(y, yo)
    num = np.linalg.norm(y.astype(np.float64) - yo, axis=1)
    den = np.linalg.norm(yo.astype(np.float64), axis=1) + 1e-30
    row = float((num / den).max())
    assert err <= TOL, f"rel Frobenius error {err}"
    assert row <= ROW_TOL, f"worst row relative error {row}"
    if bound is not None:
        diff = np.abs(y.astype(np.float64) - yo.astype(np.float64))
        lim = bound + 2.0 ** -23 * np.abs(yo.astype(np.float64))
        bad = np.argwhere(diff > lim)
        worst = float((diff / lim).max())
        assert len(bad) == 0, f"{len(bad)} outputs outside the accumulation bound (worst {worst:.2f}x), first {bad[:5]}"
    return err, row


def _layer(dqm, T, H, W, cube, Ci, Co, rank, dtype, xseed, wseed, svd="oracle", n_out=4, w_out=2, core_group=32,
           core_bits=8):
    x = synth.make_activation(T, H, W, Ci, seed=xseed, dtype=dtype, n_outliers=n_out)
    wt = synth.make_weight(Ci, Co, seed=wseed, dtype=dtype, outlier_rows=w_out)
    xf, wf = synth.to_f32_numpy(x), synth.to_f32_numpy(wt)
    if svd == "oracle" and rank > 0:
        l1, l2, _ = lowrank.svd_factors(wf, rank)
    else:
        l1, l2 = _random_factors(Ci, Co, rank, wseed + 1)
    weights = dqm.dq_prepare_weights_lowrank(wt, l1 if rank else None, l2 if rank else None, device=0)
    qa = dqm.dq_qact_create(weights, (T, H, W) + tuple(cube), core_group=core_group, core_bits=core_bits)
    xd = x.to(DEV)
    y = torch.full((T * H * W, Co), float("nan"), dtype=torch.float32, device=DEV)
    dqm.dq_linear(weights, xd, qa, y)
    torch.cuda.synchronize()
    return dict(x=xf, wt=wf, l1=l1, l2=l2, weights=weights, qa=qa, y=y.cpu().numpy(), g=cubes.Geometry(T, H, W, *cube),
                core_group=core_group, core_bits=core_bits)


def _layer_from_input(dqm, xf, dtype, grid, cube, Co, rank, wseed, core_group=32, core_bits=8):
    """Run dq_linear on the given activation (fp32 numpy [N][Ci] whose values
    are representable in `dtype`), with a seeded weight and the oracle's SVD
    factors; returns the dict _full_compare takes."""
    T, H, W = grid
    Ci = xf.shape[1]
    x = torch.from_numpy(np.ascontiguousarray(xf)).to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    assert np.array_equal(synth.to_f32_numpy(x).view(np.uint32), xf.view(np.uint32))
    wt = synth.make_weight(Ci, Co, seed=wseed, dtype=dtype, outlier_rows=2)
    wf = synth.to_f32_numpy(wt)
    l1, l2, _ = lowrank.svd_factors(wf, rank)
    weights = dqm.dq_prepare_weights_lowrank(wt, l1, l2, device=0)
    qa = dqm.dq_qact_create(weights, (T, H, W) + tuple(cube), core_group=core_group, core_bits=core_bits)
    y = torch.full((T * H * W, Co), float("nan"), dtype=torch.float32, device=DEV)
    dqm.dq_linear(weights, x.to(DEV), qa, y)
    torch.cuda.synchronize()
    return dict(x=xf, wt=wf, l1=l1, l2=l2, weights=weights, qa=qa, y=y.cpu().numpy(), g=cubes.Geometry(T, H, W, *cube),
                core_group=core_group, core_bits=core_bits)


def _full_compare(dqm, L):
    got = dqm.dq_qact_export(L["qa"])
    q = layer.quantize_activation(L["x"], L["g"], L["l1"] if L["l1"].shape[1] else None,
                                  core_group=L.get("core_group", 32), core_bits=L.get("core_bits", 8))
    assert np.array_equal(got["core_codes"], q["core_codes"]), "core codes"
    if q["core_scales"] is not None:
        assert np.array_equal(got["core_scales"], q["core_scales"]), "core scales"
    assert np.array_equal(got["delta_scales"], q["delta_scales"]), "delta scales"
    assert np.array_equal(got["delta_codes"], q["delta_codes"]), "delta codes"
    r = lowrank.residual(L["wt"], L["l1"], L["l2"])
    rc, rs = lowrank.quantize_residual(r)
    wexp = dqm.dq_weights_export(L["weights"])
    assert np.array_equal(wexp["r"].view(np.uint32), r.view(np.uint32)), "R"
    assert np.array_equal(wexp["rcodes"], rc) and np.array_equal(wexp["rscales"], rs), "Q4(R)"
    if L["l1"].shape[1]:
        _check_u(got["U"], q["U"], L["x"][q["tokens"]], L["l1"])
    else:
        q["U"] = np.zeros((len(q["tokens"]), 0), np.uint16)
    yo = layer.forward(q, L["g"], rc, rs, L["l2"])
    assert not np.isnan(L["y"]).any(), "unwritten outputs"
    bound = _abs_bound(q, L["g"], rc, rs, L["l2"], L["x"][q["tokens"]], L["l1"])
    return _check_y(L["y"], yo, bound)


