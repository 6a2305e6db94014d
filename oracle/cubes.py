"""Cube partition, core tokens and delta tokens.

DeltaQuant notes, 关键设计 2 (spatiotemporal cube partition): the flattened
activation X in R^{N x Ci}, N = T H W, is reshaped back to T x H x W x Ci and
cut into non-overlapping t x h x w cubes X^(k) in R^{thw x Ci}.
关键设计 3 (the core/delta equation): the core token of cube k is the mean of
its tokens, and every token's delta is the token minus that core (the core is
broadcast over the cube).

Readings (see the package docstring): R1 clipped partial cubes, R2 row-major
flattening and lexicographic in-cube order, R3 fp32 block-of-64 sums and one
IEEE division, R4 delta against the unquantised fp32 core.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

BLOCK = 64          # reading R3: tokens per partial sum


@dataclass(frozen=True)
class Geometry:
    T: int
    H: int
    W: int
    t: int
    h: int
    w: int

    def __post_init__(self):
        for full, c in ((self.T, self.t), (self.H, self.h), (self.W, self.w)):
            if not (full >= 1 and 1 <= c <= full):
                raise ValueError("cube extents must satisfy 1 <= t <= T etc.")

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    @property
    def grid(self):
        """Cubes along each axis (partial cubes at the high end count, R1)."""
        return (-(-self.T // self.t), -(-self.H // self.h), -(-self.W // self.w))

    @property
    def K(self) -> int:
        a, b, c = self.grid
        return a * b * c

    @property
    def S(self) -> int:
        return self.t * self.h * self.w


def cube_of_token(g: Geometry, tokens=None) -> np.ndarray:
    """Cube index of each token: n = (ti H + hi) W + wi lies in cube
    (ti // t, hi // h, wi // w), cubes numbered row-major over the cube grid."""
    n = np.arange(g.N, dtype=np.int64) if tokens is None else np.asarray(tokens, dtype=np.int64)
    ti, rem = np.divmod(n, g.H * g.W)
    hi, wi = np.divmod(rem, g.W)
    _, Hc, Wc = g.grid
    return ((ti // g.t) * Hc + hi // g.h) * Wc + wi // g.w


def cube_tokens(g: Geometry, cube_ids=None):
    """Token ids of each cube, present tokens only, in lexicographic
    (dt, dh, dw) order, padded at the end with -1; and the counts.

    Returns (table int64 [len(ids), t*h*w], counts int64 [len(ids)]).
    """
    Tc, Hc, Wc = g.grid
    ids = np.arange(g.K, dtype=np.int64) if cube_ids is None else np.asarray(cube_ids, dtype=np.int64)
    kt, rem = np.divmod(ids, Hc * Wc)
    kh, kw = np.divmod(rem, Wc)
    dt, dh, dw = (a.reshape(-1) for a in np.meshgrid(np.arange(g.t), np.arange(g.h), np.arange(g.w),
                                                     indexing="ij"))
    ti = kt[:, None] * g.t + dt[None]
    hi = kh[:, None] * g.h + dh[None]
    wi = kw[:, None] * g.w + dw[None]
    present = (ti < g.T) & (hi < g.H) & (wi < g.W)
    n = np.where(present, (ti * g.H + hi) * g.W + wi, -1)
    order = np.argsort(~present, axis=1, kind="stable")     # present first, lexicographic order kept
    return np.take_along_axis(n, order, axis=1), present.sum(axis=1)


def cube_core(x32: np.ndarray, g: Geometry, cube_ids=None, max_elems: int = 1 << 25) -> np.ndarray:
    """Core token of each requested cube, fp32 [len(ids), Ci] (关键设计 3).

    Reading R3: within a cube, tokens [64 j, 64 j + 64) of the lexicographic
    list are summed one after the other in fp32 (starting from the first
    token, not from 0); the block partials are then summed in block order in
    fp32; the total is divided by the token count with one fp32 division.
    """
    x32 = np.asarray(x32, dtype=np.float32)
    tbl, cnt = cube_tokens(g, cube_ids)
    K, S = tbl.shape
    Ci = x32.shape[1]
    nb = -(-S // BLOCK)
    padded = np.full((K, nb * BLOCK), -1, dtype=np.int64)
    padded[:, :S] = tbl
    padded = padded.reshape(K, nb, BLOCK)
    out = np.empty((K, Ci), dtype=np.float32)
    step = max(1, max_elems // max(1, nb * Ci))
    for c0 in range(0, K, step):
        blk = padded[c0:c0 + step]
        part = x32[np.maximum(blk[:, :, 0], 0)]               # first token of each block
        for j in range(1, BLOCK):
            idx = blk[:, :, j]
            valid = idx >= 0
            if not valid.any():
                break
            part = np.where(valid[..., None], part + x32[np.maximum(idx, 0)], part)
        total = part[:, 0]
        c = cnt[c0:c0 + step]
        for b in range(1, nb):
            total = np.where((c > BLOCK * b)[:, None], total + part[:, b], total)
        out[c0:c0 + step] = total / c[:, None].astype(np.float32)
    return out


def cube_delta(x32: np.ndarray, core32: np.ndarray, g: Geometry, tokens, core_row_of_cube=None) -> np.ndarray:
    """delta[n] = fl32(x[n] - core[cube(n)]) for the requested tokens (R4).

    `core32` holds the cores of some cubes; `core_row_of_cube` maps a cube id
    to its row in `core32` (identity when all cubes are present)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    k = cube_of_token(g, tokens)
    rows = k if core_row_of_cube is None else core_row_of_cube[k]
    return (np.asarray(x32, dtype=np.float32)[tokens] - core32[rows]).astype(np.float32)
