"""GPU parity of the quantizer on its edge cases, through every form of the
activation pass.

The codes and scale codes follow the quantizer of the DeltaQuant page
(关键设计 4: s = max / q_max, here the smallest power of two with
max <= q_max 2^e; round to nearest, ties to even; signs kept), applied to the
cube cores and deltas of 关键设计 3.  The HIP path encodes with the gfx950
scaled converts and passes 2^-127 (an fp32 subnormal) as the scale of
all-zero and subnormal groups; these tests feed exactly the inputs where
that could go wrong and require every code and scale code to match the
oracle bit for bit:

  const      constant cubes (8-bit significands): every delta is exactly
             +0, so each token's delta group is all zero (scale code 0);
  neg0       cubes of -0.0: core -0 (FP8 code 0x80), deltas +0;
  mixed0     random +-0: cores +0 or -0, deltas -0 (FP4 code 0x8) and +0;
  fp4mid     deltas on every FP4 grid point and midpoint of their group's
             scale, the group maximum exactly 6 2^e (cores exact multiples);
  fp4edge    zero cores, delta maxima one fp32 (or bf16) step above or below
             6 2^e, the rest on grid points and midpoints of both scales;
  fp8mid     constant cubes whose cores sit on FP8 E4M3 midpoints (normal
             and subnormal) and one step either side, maximum 448 2^e;
  fp8edge    the same with the maximum just above 448 2^e (next scale up);
  subnormal  fp32 (or bf16) subnormal tokens: subnormal cube sums, means,
             deltas and group maxima (scale code 0);
  tinynormal tokens just above the normal threshold (clamped exponents);
  random     ordinary Gaussian tokens.

The scenario of a 32-channel group changes from cube to cube, so every cube
holds several.  Deltas of the constructed cubes come in adjacent pairs
(d, -d) in the cube's token order (a token left over is the core itself), so
the ordered fp32 sums are exact and the core is the intended value.

Forms of the activation pass, chosen by the cube size S: one-token cubes;
one pass (S = 2, 4, 9); eighths (S = 8); one wave per cube (S = 12, 16);
two phases with channel pairs (S = 32) and single channels (S = 64); the
partial-sum pass (S > 64, one frame segment and two).  Each runs with fp32
and bf16 input and with FP8 cores (groups of 32 and 64), FP4 cores and bf16
cores.
"""
import numpy as np
import pytest

from oracle import cubes, mx
from parity_util import _full_compare, _layer_from_input, _say

pytestmark = pytest.mark.gpu

SCEN = ("const", "neg0", "mixed0", "fp4mid", "fp4edge", "fp8mid", "fp8edge", "subnormal", "tinynormal", "random")

# FP4 grid points and midpoints in units of 2^(e-2) (values 0 .. 6 times 2^e)
FP4_UNITS = np.array([0, 1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 14, 16, 20, 24], dtype=np.float64)


def _fp8_pool():
    """E4M3 magnitudes to place cores on: normal grid points, midpoints and
    the values one 2^-7 either side of a midpoint, subnormal grid points and
    midpoints; all at most 448 and at most 8 significant bits."""
    vals = []
    for kk in range(-6, 9):
        for m in range(8):
            mid = 1 + (2 * m + 1) / 16
            vals += [(1 + m / 8) * 2.0 ** kk, mid * 2.0 ** kk, (mid + 2 ** -7) * 2.0 ** kk,
                     (mid - 2 ** -7) * 2.0 ** kk]
    vals += [j * 2.0 ** -9 for j in range(8)] + [(2 * j + 1) * 2.0 ** -10 for j in range(8)]
    v = np.array(vals)
    return v[v <= 448.0]


FP8_POOL = _fp8_pool()


def _signs(rng, shape):
    return np.where(rng.random(shape) < 0.5, -1.0, 1.0)


def _pairs(n, rng, draw):
    """n rows of 32 deltas: adjacent rows (2p, 2p + 1) hold d and -d (one
    draw() per pair); an odd last row is zero."""
    d = np.zeros((n, 32))
    for p in range(n // 2):
        v = draw()
        d[2 * p], d[2 * p + 1] = v, -v
    return d


def _group(sc, n, rng, bf16):
    """Values of one cube's 32-channel group: n rows."""
    if sc == "const":
        c = _signs(rng, 32) * rng.integers(128, 256, 32) * np.ldexp(1.0, rng.integers(-40, 20, 32))
        return np.tile(c, (n, 1))
    if sc == "neg0":
        return np.full((n, 32), -0.0)
    if sc == "mixed0":
        return np.where(rng.random((n, 32)) < 0.5, -0.0, 0.0)
    if sc == "fp4mid":
        e = int(rng.integers(-12, 8))
        u = 2.0 ** (e - 2)
        c = rng.integers(-100, 101, 32) * u

        def draw():
            v = _signs(rng, 32) * FP4_UNITS[rng.integers(0, len(FP4_UNITS), 32)]
            v[rng.integers(0, 32)] = 24 * _signs(rng, 1)[0]          # group maximum exactly 6 2^e
            return v * u
        return c + _pairs(n, rng, draw)
    if sc == "fp4edge":
        e = int(rng.integers(-12, 8))
        above = bool(rng.integers(0, 2))
        top = 6.0 * 2.0 ** e
        if bf16:
            edge = (1.5 + (2 ** -7 if above else -2 ** -7)) * 2.0 ** (e + 2)
        else:
            edge = float(np.nextafter(np.float32(top), np.float32(np.inf if above else 0)))
        pool = np.array([0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5] + ([6] if above else []))

        def draw():
            v = _signs(rng, 32) * pool[rng.integers(0, len(pool), 32)] * 2.0 ** e
            v[rng.integers(0, 32)] = edge * _signs(rng, 1)[0]
            return v
        return _pairs(n, rng, draw)
    if sc in ("fp8mid", "fp8edge"):
        e = int(rng.integers(-24, 12))
        c = _signs(rng, 32) * FP8_POOL[rng.integers(0, len(FP8_POOL), 32)]
        c[rng.integers(0, 32)] = (448.0 if sc == "fp8mid" else (1.75 + 2 ** -7) * 256) * _signs(rng, 1)[0]
        return np.tile(c * 2.0 ** e, (n, 1))
    if sc == "subnormal":
        if bf16:
            return rng.integers(-127, 128, (n, 32)) * 2.0 ** -133
        return rng.integers(-(1 << 22), 1 << 22, (n, 32)) * 2.0 ** -149
    if sc == "tinynormal":
        v = _signs(rng, (n, 32)) * (1 + rng.random((n, 32))) * np.ldexp(1.0, rng.integers(-126, -118, (n, 32)))
    else:
        v = rng.standard_normal((n, 32))
    v = v.astype(np.float32).astype(np.float64)
    return mx.bf16_bits_to_f64(mx.f64_to_bf16_bits(v)) if bf16 else v


def edge_activation(g, Ci, dtype, seed):
    """X [N][Ci] fp32 (values representable in `dtype`) built cube by cube."""
    rng = np.random.default_rng(seed)
    bf16 = dtype == "bf16"
    x = np.zeros((g.N, Ci), np.float64)
    tbl, cnt = cubes.cube_tokens(g)
    for k in range(g.K):
        toks = tbl[k, :cnt[k]]
        for gi in range(Ci // 32):
            x[toks, 32 * gi:32 * gi + 32] = _group(SCEN[(gi + 3 * k) % len(SCEN)], len(toks), rng, bf16)
    x32 = x.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64).view(np.uint64), x.view(np.uint64)), "edge input not fp32"
    if bf16:
        b = mx.bf16_bits_to_f64(mx.f32_to_bf16_bits(x32))
        assert np.array_equal(b.view(np.uint64), x.view(np.uint64)), "edge input not representable in bf16"
    return x32


GEOMS = [
    (2, 5, 8, (1, 1, 1)),       # one-token cubes
    (2, 4, 6, (1, 1, 2)),       # one pass, 2-token cubes
    (3, 5, 7, (1, 2, 2)),       # one pass, 4-token cubes, clipped
    (3, 6, 6, (1, 3, 3)),       # one pass, 9-token cubes (7 per block)
    (3, 6, 8, (2, 2, 2)),       # eighths, second frame segment
    (3, 6, 8, (1, 3, 4)),       # one wave per cube, 12 tokens
    (3, 8, 8, (1, 4, 4)),       # one wave per cube, 16 tokens
    (4, 8, 8, (2, 4, 4)),       # two phases, channel pairs (32 tokens)
    (5, 8, 16, (4, 2, 8)),      # two phases, single channels (64 tokens), second frame segment
    (3, 9, 10, (3, 9, 10)),     # partial-sum pass, one global cube of 270 tokens
    (5, 9, 10, (4, 9, 10)),     # partial-sum pass in both frame segments
]
CORES = [(8, 32), (8, 64), (4, 32), (16, 32)]
CASES = [(geo, dt, cb, cg) for geo in GEOMS for dt in ("f32", "bf16") for cb, cg in CORES]


def _id(c):
    (T, H, W, cube), dt, cb, cg = c
    return f"{T}x{H}x{W}_c{'x'.join(map(str, cube))}_{dt}_core{cb}g{cg}"


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_encoder_edges(dqm, case):
    (T, H, W, cube), dtype, core_bits, core_group = case
    Ci, Co, rank = 192, 64, 16
    _say(f"case encoder edges {_id(case)}")
    g = cubes.Geometry(T, H, W, *cube)
    seed = 7000 + GEOMS.index((T, H, W, cube)) * 10 + (dtype == "bf16")
    xf = edge_activation(g, Ci, dtype, seed)
    L = _layer_from_input(dqm, xf, dtype, (T, H, W), cube, Co, rank, wseed=seed + 1, core_group=core_group,
                          core_bits=core_bits)
    err, row = _full_compare(dqm, L)
    _say(f"encoder edges {_id(case)}: codes bit-exact; rel err {err:.2e} worst row {row:.2e}")


@pytest.fixture(scope="module")
def dqm(lib):
    from w4a4_quantized_linear_cube_amd import dq
    return dq
