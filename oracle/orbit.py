"""OrbitQuant-style W4A4 front end: the online RPBH rotation and the
Lloyd-Max codebook quantizer (the OrbitQuant page: 方法 / 核心思路, 离线的权重量化,
在线的激活量化).

What the page fixes: activations are projected by a random permuted block
Hadamard transform (RPBH) onto a normalized rotated basis, in which every
coordinate follows about the same standard (near-Gaussian) law, so one
precomputed Lloyd-Max codebook serves every timestep, prompt and layer; each
rotated coordinate is quantized to its nearest codebook entry.  Weights are
rotated by the same matrix offline and quantized row by row in the rotated
basis, so the rotation cancels inside the layer: (x R^T)(w R^T)^T = x w^T.

Readings taken where the page is silent (the plainest ones):
  O1  RPBH = a permutation P of the Ci channels (an input: drawn by the
      caller), then the orthonormal Walsh-Hadamard transform on consecutive
      blocks of b = 256 channels: x' = blockdiag(H_b / sqrt(b)) x[P].
      sqrt(256) = 16, so the normalization is exact.  The transform is the
      radix-2 butterfly network in fp32: stages h = 1, 2, 4, .., b/2, each
      replacing (u, v) = (x[i], x[i + h]) by (u + v, u - v) for every i with
      i & h == 0, then the multiplication by 1/16.
  O2  "normalized basis": each rotated row (token, or output channel of the
      weight) is divided by its RMS s = sqrt(sum x'^2 / Ci), so its
      coordinates are about N(0, 1); s is kept in fp32 and multiplies the
      output.  The sum of squares is taken in fp32, per 256-channel block in
      channel order, then over the blocks in order; s = sqrt(sum / Ci) with
      IEEE division and square root.  A zero row has s = 0 and codes as
      coordinates of 0.
  O3  the codebook is the Lloyd-Max quantizer of N(0, 1) with 2^bits levels
      (the fixed point of: boundaries at midpoints of neighbouring levels,
      levels at the conditional means of their cells), each level rounded to
      bf16, the input type of the matrix cores that contract the decoded
      values (the codebook is not a float format, so no scaled-MFMA format
      can take the codes directly).
  O4  a coordinate v = fl32(x' / s) takes the index of the nearest bf16
      level; an exact tie (v on the midpoint of two levels) takes the even
      index.  Codes are level indices 0 .. 2^bits - 1 in ascending order,
      stored two per byte (even channel in the low nibble).
  O5  y[n, j] = fl32(fl32(acc[n, j] * s_x[n]) * s_w[j]) with acc the exact
      sum over channels of level(x code) * level(w code).  No low-rank
      branch (the page names none).
"""
from __future__ import annotations

import math

import numpy as np

from . import mx

BLOCK = 256


# ------------------------------------------------------------ codebook ----
def _phi(t):
    return math.exp(-0.5 * t * t) / math.sqrt(2.0 * math.pi) if math.isfinite(t) else 0.0


def _Phi(t):
    if t == math.inf:
        return 1.0
    if t == -math.inf:
        return 0.0
    return 0.5 * (1.0 + math.erf(t / math.sqrt(2.0)))


def lloyd_max_gaussian(levels: int, iters: int = 20000, tol: float = 1e-15) -> np.ndarray:
    """Lloyd-Max quantizer of the standard normal with `levels` levels
    (ascending, fp64): iterate t_i = (y_i + y_{i+1}) / 2 and
    y_i = E[X | t_{i-1} < X <= t_i] = (phi(t_{i-1}) - phi(t_i)) / (Phi(t_i) - Phi(t_{i-1}))
    from equally spaced quantiles until nothing moves."""
    y = np.array([math.sqrt(2.0) * _erfinv(2.0 * (i + 0.5) / levels - 1.0) for i in range(levels)])
    for _ in range(iters):
        t = np.concatenate([[-math.inf], (y[:-1] + y[1:]) / 2.0, [math.inf]])
        new = np.array([(_phi(t[i]) - _phi(t[i + 1])) / (_Phi(t[i + 1]) - _Phi(t[i])) for i in range(levels)])
        done = np.max(np.abs(new - y)) <= tol
        y = new
        if done:
            break
    return y


def _erfinv(z: float) -> float:
    """Inverse error function by Newton's method on math.erf (start values
    only; the Lloyd iteration removes any error in them)."""
    x = 0.0
    for _ in range(100):
        x -= (math.erf(x) - z) / (2.0 / math.sqrt(math.pi) * math.exp(-x * x))
    return x


def codebook_bf16(bits: int) -> np.ndarray:
    """The O3 codebook: bf16 bits (uint16) of the 2^bits Lloyd-Max levels."""
    return mx.f64_to_bf16_bits(lloyd_max_gaussian(1 << bits))


# ------------------------------------------------------------ rotation ----
def fwht_blocks(x32: np.ndarray, b: int = BLOCK) -> np.ndarray:
    """O1's orthonormal block Walsh-Hadamard transform along the last axis,
    fp32 butterflies stage by stage, then the exact 1/sqrt(b) scaling."""
    x = np.array(x32, dtype=np.float32, copy=True)
    C = x.shape[-1]
    if C % b:
        raise ValueError("channel count must be a multiple of the block size")
    v = x.reshape(x.shape[:-1] + (C // b, b))
    h = 1
    while h < b:
        w = v.reshape(v.shape[:-1] + (b // (2 * h), 2, h))
        u, t = w[..., 0, :].copy(), w[..., 1, :].copy()
        w[..., 0, :] = u + t
        w[..., 1, :] = u - t
        h *= 2
    lg = int(round(math.log2(b)))
    if (1 << lg) != b or lg % 2:
        raise ValueError("the block size must be a power of four (exact 1/sqrt(b))")
    scale = np.float32(2.0 ** (-lg // 2))
    return (v * scale).reshape(x.shape).astype(np.float32)


def rpbh(x32: np.ndarray, perm: np.ndarray, b: int = BLOCK) -> np.ndarray:
    """x' = blockdiag(H_b / sqrt(b)) x[P] (O1)."""
    return fwht_blocks(np.asarray(x32, dtype=np.float32)[..., np.asarray(perm, dtype=np.int64)], b)


def rms_scale(xr32: np.ndarray, b: int = BLOCK) -> np.ndarray:
    """O2: s = sqrt(sum x'^2 / Ci), fp32, the sum per block in channel order
    then over blocks in order."""
    x = np.asarray(xr32, dtype=np.float32)
    C = x.shape[-1]
    v = x.reshape(x.shape[:-1] + (C // b, b))
    sq = v * v                                        # fl32 squares
    part = sq[..., 0].copy()
    for i in range(1, b):
        part = part + sq[..., i]
    tot = part[..., 0].copy()
    for j in range(1, C // b):
        tot = tot + part[..., j]
    return np.sqrt(tot / np.float32(C)).astype(np.float32)


def nearest_level(v32: np.ndarray, cb_bits: np.ndarray) -> np.ndarray:
    """O4: index of the nearest bf16 level, exact ties to the even index."""
    lv = mx.bf16_bits_to_f64(cb_bits)              # ascending
    v = np.asarray(v32, dtype=np.float64)
    mids = (lv[:-1] + lv[1:]) / 2.0                # exact in fp64
    idx = np.searchsorted(mids, v, side="left")    # midpoints strictly below v
    at = (idx < len(mids)) & (v == mids[np.minimum(idx, len(mids) - 1)])
    return np.where(at & (idx % 2 == 1), idx + 1, idx).astype(np.uint8)


def quantize_rows(x32: np.ndarray, perm: np.ndarray, cb_bits: np.ndarray, b: int = BLOCK) -> dict:
    """Rotate, normalize and code rows (tokens, or output channels of W^T).
    Returns the rotated rows, their scales, codes [rows][Ci] (one per byte)
    and packed codes [rows][Ci/2]."""
    xr = rpbh(x32, perm, b)
    s = rms_scale(xr, b)
    safe = np.where(s > 0, s, np.float32(1.0))
    v = np.where(s[..., None] > 0, (xr / safe[..., None]).astype(np.float32), np.float32(0.0))
    codes = nearest_level(v, cb_bits)
    return dict(rot=xr, scale=s, codes=codes, packed=mx.pack_fp4(codes))


def forward(qx: dict, qw: dict, cbx_bits: np.ndarray, cbw_bits: np.ndarray) -> np.ndarray:
    """O5: y = fl32(fl32(acc s_x) s_w), acc = sum_c level(x) level(w) (fp64, exact)."""
    lx = mx.bf16_bits_to_f64(cbx_bits)[qx["codes"]]
    lw = mx.bf16_bits_to_f64(cbw_bits)[qw["codes"]]
    acc = (lx @ lw.T).astype(np.float32)
    return ((acc * qx["scale"][:, None]).astype(np.float32) * qw["scale"][None, :]).astype(np.float32)
