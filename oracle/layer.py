"""The delta-W4A4 layer, end to end, on the CPU.

DeltaQuant notes, 关键设计 4 (the three-term equation):
    X^(k) W  ~  X^(k) L1 L2  +  Q8(core_k) Q4(R)  +  Q4(delta^(k)) Q4(R)
The core term is computed once per cube and broadcast to the cube's tokens
(the "dynamic token bias" of the same section).  Quantizers: FP8 for cores,
FP4 for deltas and R, MX block scales (readings R5-R8); the low-rank branch
in bf16 with fp32 output (R10).  Sums and products are formed in fp64, and the
output is rounded once to fp32.
"""
from __future__ import annotations

import numpy as np

from . import cubes, mx


def quantize_activation(x32: np.ndarray, g: cubes.Geometry, l1_bits: np.ndarray, cube_ids=None, tokens=None,
                        core_group: int = 32, core_bits: int = 8) -> dict:
    """What the activation pass produces, for the given cubes (all by default).

    Cores are always formed from every token of a cube; deltas and U are
    formed for `tokens` (default: all tokens of the given cubes), which must
    lie in those cubes.

    Returns a dict with
      cube_ids [k]; tokens [n] (ascending);
      core [k, Ci] fp32; core_codes [k, Ci] and core_scales [k, Ci/32] (FP8,
      or FP4 for core_bits = 4, the 4-bit point of the pages' core-precision
      ablation; one exponent per core_group channels: 32, or the pages' 64;
      for core_bits = 16 the bf16 bits of the core, round to nearest even,
      and no scales); core_fmt;
      delta [n, Ci] fp32; delta_codes [n, Ci/2] packed and delta_scales
      [n, Ci/32] (FP4); U [n, r] bf16 bits.
    """
    x32 = np.asarray(x32, dtype=np.float32)
    ids = np.arange(g.K, dtype=np.int64) if cube_ids is None else np.asarray(cube_ids, dtype=np.int64)
    core = cubes.cube_core(x32, g, ids)
    if tokens is None:
        tbl, _ = cubes.cube_tokens(g, ids)
        tokens = np.sort(tbl[tbl >= 0])
    else:
        tokens = np.sort(np.asarray(tokens, dtype=np.int64))
        if not np.all(np.isin(cubes.cube_of_token(g, tokens), ids)):
            raise ValueError("tokens outside the given cubes")
    row_of_cube = np.full(g.K, -1, dtype=np.int64)
    row_of_cube[ids] = np.arange(len(ids))
    delta = cubes.cube_delta(x32, core, g, tokens, row_of_cube)
    core_fmt = {8: "fp8", 4: "fp4", 16: "bf16"}[core_bits]
    if core_fmt == "bf16":
        core_codes, core_scales = mx.f32_to_bf16_bits(core), None
    else:
        core_codes, core_scales = mx.mx_quantize(core, core_fmt, core_group)
    d_codes, d_scales = mx.mx_quantize(delta, "fp4")
    out = dict(cube_ids=ids, tokens=tokens, row_of_cube=row_of_cube, core=core,
               core_codes=core_codes, core_scales=core_scales, core_fmt=core_fmt, delta=delta,
               delta_codes=mx.pack_fp4(d_codes), delta_scales=d_scales)
    if l1_bits is not None:
        out["U"] = low_rank_down(x32[tokens], l1_bits)
    return out


def low_rank_down(x32_rows: np.ndarray, l1_bits: np.ndarray) -> np.ndarray:
    """U = bf16( bf16(x) L1 ), the sum in fp64 (R10).  Returns bf16 bits."""
    xb = mx.bf16_bits_to_f64(mx.f32_to_bf16_bits(x32_rows))
    return mx.f64_to_bf16_bits(xb @ mx.bf16_bits_to_f64(l1_bits))


def assemble(lr: np.ndarray, core_term: np.ndarray, delta_term: np.ndarray, core_rows: np.ndarray) -> np.ndarray:
    """Y = fl32(LR + core_term[cube(n)] + delta_term): the three terms of the
    three-term equation, the core term broadcast from its cube."""
    return (lr + core_term[core_rows] + delta_term).astype(np.float32)


def forward(q: dict, g: cubes.Geometry, r_codes: np.ndarray, r_scales: np.ndarray, l2_bits: np.ndarray,
            rows=None) -> np.ndarray:
    """fp32 output for the tokens of `q` (or the subset `rows` of q['tokens'],
    given as positions into it).  `r_codes` [Co][Ci/2] packed FP4 and
    `r_scales` [Co][Ci/32] hold Q4(R)."""
    sel = slice(None) if rows is None else np.asarray(rows)
    tokens = q["tokens"][sel]
    rdq = mx.mx_dequantize(mx.unpack_fp4(r_codes), r_scales, "fp4").T          # [Ci][Co]
    core_dq = core_values(q)                                                        # [k][Ci]
    delta_dq = mx.mx_dequantize(mx.unpack_fp4(q["delta_codes"][sel]), q["delta_scales"][sel], "fp4")
    lr = mx.bf16_bits_to_f64(q["U"][sel]) @ mx.bf16_bits_to_f64(l2_bits)
    core_rows = q["row_of_cube"][cubes.cube_of_token(g, tokens)]
    return assemble(lr, core_dq @ rdq, delta_dq @ rdq, core_rows)


# ------------------------------------------------------------ sanity ----
def core_values(q: dict) -> np.ndarray:
    """The quantized cores' values in fp64 (exact), whatever their format."""
    fmt = q.get("core_fmt", "fp8")
    if fmt == "bf16":
        return mx.bf16_bits_to_f64(q["core_codes"])
    return mx.mx_dequantize(q["core_codes"], q["core_scales"], fmt)


def exact_output(x32_rows: np.ndarray, wt32: np.ndarray) -> np.ndarray:
    """X W in fp64 (W = wt32^T)."""
    return np.asarray(x32_rows, dtype=np.float64) @ np.asarray(wt32, dtype=np.float64).T


def direct_output(x32_rows: np.ndarray, u_bits: np.ndarray, l2_bits: np.ndarray, r_codes, r_scales) -> np.ndarray:
    """Direct W4A4 with the same low-rank branch: LR + Q4(X) Q4(R), X quantized
    per token with the same MX-FP4 rule and no cubes."""
    xc, xs = mx.mx_quantize(np.asarray(x32_rows, dtype=np.float32), "fp4")
    rdq = mx.mx_dequantize(mx.unpack_fp4(r_codes), r_scales, "fp4").T
    lr = mx.bf16_bits_to_f64(u_bits) @ mx.bf16_bits_to_f64(l2_bits)
    return (lr + mx.mx_dequantize(xc, xs, "fp4") @ rdq).astype(np.float32)


def rtn_output(x32_rows: np.ndarray, wt32: np.ndarray) -> np.ndarray:
    """Plain W4A4 round-to-nearest, no low-rank branch: Q4(X) Q4(W)."""
    xc, xs = mx.mx_quantize(np.asarray(x32_rows, dtype=np.float32), "fp4")
    wc, ws = mx.mx_quantize(np.asarray(wt32, dtype=np.float32), "fp4")
    return (mx.mx_dequantize(xc, xs, "fp4") @ mx.mx_dequantize(wc, ws, "fp4").T).astype(np.float32)


def rel_fro(a: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    n = np.linalg.norm(ref)
    d = np.linalg.norm(np.asarray(a, dtype=np.float64) - ref)
    return float(d / n) if n > 0 else float(d)
