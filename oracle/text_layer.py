"""The 6-bit linear layers on text tokens (the cross-attention K/V
projections).

DeltaQuant notes, 损失函数/训练策略 (the implementation paragraph): every
linear layer is quantized to 4 bits except the cross-attention K and V
projections, which act only on the text tokens, cost little, and are kept at
6 bits.  Readings taken (the pages give no more):
  T1  "6-bit" is W6A6 in an MX 6-bit float: each group of 32 consecutive
      channels of a token (and of an output channel of R) shares one E8M0
      power-of-two scale, chosen by the quantizer of 关键设计 4 (smallest 2^e
      with max <= q_max 2^e, R5) with q_max the format's largest value, and
      elements round to nearest, ties to even (R7).  Format E2M3 (q_max 7.5)
      or E3M2 (q_max 28); the pages name neither.
  T2  text tokens have no (T, H, W) grid, so there are no cubes, cores or
      deltas: the activation is quantized directly, X -> Q6(X).
  T3  the weight keeps the SVDQuant split of 关键设计 4 (the same engine and
      rank for every quantized layer): W = L1 L2 + R, R -> Q6(R), and the
      low-rank branch U = bf16(bf16(X) L1) of reading R10.
So, for token n:  y_n = U_n L2 + Q6(x_n) Q6(R), sums in fp64, output fp32.
"""
from __future__ import annotations

import numpy as np

from . import layer, mx


def quantize_text_activation(x32: np.ndarray, l1_bits, fmt: str) -> dict:
    """Q6(X) per token (T1, T2) and U (T3).  Returns codes [N][Ci] (one per
    byte), packed codes [N][3 Ci/4], scale codes [N][Ci/32], U bits [N][r]."""
    x32 = np.asarray(x32, dtype=np.float32)
    codes, scales = mx.mx_quantize(x32, fmt)
    out = dict(fmt=fmt, codes=codes, packed=mx.pack_fp6(codes), scales=scales)
    if l1_bits is not None:
        out["U"] = layer.low_rank_down(x32, l1_bits)
    return out


def forward(q: dict, r_packed: np.ndarray, r_scales: np.ndarray, l2_bits) -> np.ndarray:
    """y = U L2 + Q6(X) Q6(R) (fp64 sums, one rounding to fp32).
    `r_packed` [Co][3 Ci/4] and `r_scales` [Co][Ci/32] hold Q6(R)."""
    fmt = q["fmt"]
    rdq = mx.mx_dequantize(mx.unpack_fp6(r_packed), r_scales, fmt).T          # [Ci][Co]
    xdq = mx.mx_dequantize(q["codes"], q["scales"], fmt)                        # [N][Ci]
    y = xdq @ rdq
    if l2_bits is not None and np.asarray(l2_bits).shape[0]:
        y = y + mx.bf16_bits_to_f64(q["U"]) @ mx.bf16_bits_to_f64(l2_bits)
    return y.astype(np.float32)
