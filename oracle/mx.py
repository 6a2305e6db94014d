"""Number formats of the oracle: FP4 E2M1, FP8 E4M3, E8M0 scales, bf16.

Quantizer (DeltaQuant notes, 关键设计 4, the quantizer definition): a group
X is stored as round(X / s) with s = max|X| / q_max, q_max = 6 for 4-bit
floats.  With MX block scales the scale must be a power of two, so s is taken
as the smallest 2^e that still satisfies max|X| <= q_max * 2^e (reading R5),
and round() is round-to-nearest with ties to the even code (reading R7).

Every value table here is built by decoding each bit pattern from the format's
own definition (sign, exponent field, mantissa field, bias).
"""
from __future__ import annotations

import numpy as np

FP4_QMAX = 6.0      # 关键设计 4: q_max = 6 for 4-bit floats
FP8_QMAX = 448.0    # reading R6: largest finite OCP E4M3 value
FP6_E2M3_QMAX = 7.5   # 6-bit floats (the 6-bit K/V projections): largest finite
FP6_E3M2_QMAX = 28.0  #   values of the OCP MX FP6 formats E2M3 and E3M2
GROUP = 32          # reading R5: MX block of 32 consecutive channels
E_MIN, E_MAX = -127, 127


def fp4_decode_magnitude(code: int) -> float:
    """E2M1, exponent bias 1: E = 0 is subnormal (M * 0.5)."""
    E, M = (code >> 1) & 3, code & 1
    if E == 0:
        return M * 0.5
    return (1.0 + M / 2.0) * 2.0 ** (E - 1)


def fp8_decode_magnitude(code: int) -> float:
    """OCP E4M3, exponent bias 7, no infinities; E=15,M=7 is NaN."""
    E, M = (code >> 3) & 15, code & 7
    if E == 15 and M == 7:
        return float("nan")
    if E == 0:
        return (M / 8.0) * 2.0 ** -6
    return (1.0 + M / 8.0) * 2.0 ** (E - 7)


def fp6_decode_magnitude(code: int, ebits: int) -> float:
    """OCP MX FP6: E2M3 (ebits 2, bias 1) or E3M2 (ebits 3, bias 3); no
    infinities or NaN; E = 0 is subnormal."""
    mbits = 5 - ebits
    bias = (1 << (ebits - 1)) - 1
    E, M = (code >> mbits) & ((1 << ebits) - 1), code & ((1 << mbits) - 1)
    if E == 0:
        return (M / 2.0 ** mbits) * 2.0 ** (1 - bias)
    return (1.0 + M / 2.0 ** mbits) * 2.0 ** (E - bias)


# magnitudes indexed by the code with its sign bit cleared, ascending
FP4_MAGS = np.array([fp4_decode_magnitude(c) for c in range(8)], dtype=np.float64)
FP8_MAGS = np.array([fp8_decode_magnitude(c) for c in range(127)], dtype=np.float64)
FP6_E2M3_MAGS = np.array([fp6_decode_magnitude(c, 2) for c in range(32)], dtype=np.float64)
FP6_E3M2_MAGS = np.array([fp6_decode_magnitude(c, 3) for c in range(32)], dtype=np.float64)
_FORMATS = {
    "fp4": (FP4_MAGS, FP4_QMAX, 3),
    "fp8": (FP8_MAGS, FP8_QMAX, 7),
    "fp6_e2m3": (FP6_E2M3_MAGS, FP6_E2M3_QMAX, 5),
    "fp6_e3m2": (FP6_E3M2_MAGS, FP6_E3M2_QMAX, 5),
}


def mx_exponent(amax, qmax: float) -> np.ndarray:
    """Smallest integer e with amax <= qmax * 2^e, clamped to [-127, 127].

    A log2 estimate is corrected with exact comparisons against qmax * 2^e
    (products of a small integer-valued float and a power of two are exact in
    fp64), so the result is the definition itself, not the estimate.
    """
    a = np.asarray(amax, dtype=np.float64)
    with np.errstate(divide="ignore"):
        est = np.where(a > 0, np.ceil(np.log2(np.where(a > 0, a, 1.0) / qmax)), E_MIN)
    e = np.clip(est, E_MIN - 2, E_MAX + 2).astype(np.int64)
    for _ in range(3):   # make qmax*2^e >= a
        e = np.where(a > np.ldexp(qmax, e), e + 1, e)
    for _ in range(3):   # and qmax*2^(e-1) < a
        e = np.where(a <= np.ldexp(qmax, e - 1), e - 1, e)
    return np.clip(e, E_MIN, E_MAX)


def round_to_grid(v: np.ndarray, mags: np.ndarray) -> np.ndarray:
    """Index of the nearest magnitude in `mags` to |v|; on an exact tie the
    even index (even mantissa) wins.  |v| must not exceed mags[-1]."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    if a.size and not np.all(a <= mags[-1]):
        raise ValueError("value outside the format's range")
    mids = (mags[:-1] + mags[1:]) / 2.0           # exact in fp64
    idx = np.searchsorted(mids, a, side="left")   # number of midpoints strictly below |v|
    at_mid = (idx < len(mids)) & (a == mids[np.minimum(idx, len(mids) - 1)])
    idx = np.where(at_mid & ((idx + 1) % 2 == 0), idx + 1, idx)
    return idx.astype(np.uint8)


def mx_quantize(x32: np.ndarray, fmt: str, scale_group: int = GROUP):
    """MX-quantize fp32 values along the last axis in groups of 32.

    Returns (codes uint8 [..., C] one code per element, scale codes uint8
    [..., C/32]).  Each group: e = mx_exponent(max|x|), element code =
    round_to_grid(x / 2^e) with the sign bit copied from x.

    scale_group = 64 takes e from the maximum over each 64 consecutive
    channels (the pages' per-group FP8 core, group size 64: 损失函数/训练策略)
    and stores it as the scale code of both of its 32-channel blocks.
    """
    mags, qmax, sign_shift = _FORMATS[fmt]
    x32 = np.asarray(x32, dtype=np.float32)
    C = x32.shape[-1]
    if C % GROUP:
        raise ValueError("channel count must be a multiple of 32")
    if scale_group not in (GROUP, 2 * GROUP) or C % scale_group:
        raise ValueError("scale group must be 32 or 64 and divide the channel count")
    g = x32.reshape(x32.shape[:-1] + (C // GROUP, GROUP))
    gs = x32.reshape(x32.shape[:-1] + (C // scale_group, scale_group))
    e = np.repeat(mx_exponent(np.abs(gs).max(axis=-1), qmax), scale_group // GROUP, axis=-1)
    v = g.astype(np.float64) * np.ldexp(1.0, -e)[..., None]     # exact
    idx = round_to_grid(v, mags)
    codes = idx | (np.signbit(g).astype(np.uint8) << sign_shift)
    return codes.reshape(x32.shape).astype(np.uint8), (e + 127).astype(np.uint8)


def mx_dequantize(codes: np.ndarray, scale_codes: np.ndarray, fmt: str) -> np.ndarray:
    """fp64 values code_value * 2^(scale - 127) (exact)."""
    mags, _, sign_shift = _FORMATS[fmt]
    codes = np.asarray(codes, dtype=np.uint8)
    mag = mags[codes & ((1 << sign_shift) - 1)]
    val = np.where((codes >> sign_shift) & 1, -mag, mag)
    C = codes.shape[-1]
    g = val.reshape(codes.shape[:-1] + (C // GROUP, GROUP))
    e = np.asarray(scale_codes, dtype=np.int64) - 127
    return (g * np.ldexp(1.0, e)[..., None]).reshape(codes.shape)


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """Two FP4 codes per byte, the even channel in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def pack_fp6(codes: np.ndarray) -> np.ndarray:
    """Six bits per code, packed little-endian in order: code i of a row at
    bits [6 i, 6 i + 6) of the row's byte string (four codes per three
    bytes, 24 bytes per 32-code MX block)."""
    c = np.asarray(codes, dtype=np.uint32)
    if c.shape[-1] % 4:
        raise ValueError("code count must be a multiple of 4")
    q = c.reshape(c.shape[:-1] + (c.shape[-1] // 4, 4))
    word = q[..., 0] | (q[..., 1] << 6) | (q[..., 2] << 12) | (q[..., 3] << 18)
    b = np.stack([word & 255, (word >> 8) & 255, (word >> 16) & 255], axis=-1)
    return b.reshape(c.shape[:-1] + (c.shape[-1] // 4 * 3,)).astype(np.uint8)


def unpack_fp6(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint32)
    t = p.reshape(p.shape[:-1] + (p.shape[-1] // 3, 3))
    word = t[..., 0] | (t[..., 1] << 8) | (t[..., 2] << 16)
    q = np.stack([(word >> (6 * i)) & 63 for i in range(4)], axis=-1)
    return q.reshape(p.shape[:-1] + (p.shape[-1] // 3 * 4,)).astype(np.uint8)


# ---------------------------------------------------------------- bf16 ----
def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even), returned as uint16 bits.

    bf16 keeps fp32's exponent range with 8 significant bits: for
    x = m 2^k (frexp, m in [0.5, 1)) its grid spacing is 2^(k - 8) for
    normal values (|x| >= 2^-126, k >= -125), and the fixed subnormal
    spacing 2^-133 below that.  rint(x / spacing) rounds to that grid with
    ties to even.  Finite inputs below the bf16 overflow threshold.
    """
    x = np.asarray(x32, dtype=np.float64)
    return f64_to_bf16_bits(x)


def f64_to_bf16_bits(x64: np.ndarray) -> np.ndarray:
    x = np.asarray(x64, dtype=np.float64)
    _, k = np.frexp(x)
    q = np.maximum(k, -125) - 8                        # log2 of the grid spacing at x
    r = np.ldexp(np.rint(np.ldexp(x, -q)), q)          # exact: <= 9 significant bits
    bits = r.astype(np.float32).view(np.uint32)        # exact: r lies on the bf16 grid
    sign = np.signbit(x).astype(np.uint32) << 31       # keeps -0 (and values that round to -0)
    return (((bits & 0x7FFFFFFF) | sign) >> 16).astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
