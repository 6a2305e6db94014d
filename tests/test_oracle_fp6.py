"""Pins of the oracle's 6-bit formats and of the 6-bit text-token layer
(DeltaQuant notes, 损失函数/训练策略: the cross-attention K/V projections are
kept at 6 bits): the OCP MX FP6 grids and their tie table, brute-force
nearest-code search, brute-force scale search, the bit order of the packing,
a lossless round trip, and a scalar re-derivation of the whole layer."""
import math

import numpy as np
import pytest

from oracle import layer, lowrank, mx, text_layer
from test_oracle_formats import _brute_exponent, _brute_nearest, _interesting_values, _read_golden

FMTS = {"fp6_e2m3": (mx.FP6_E2M3_MAGS, mx.FP6_E2M3_QMAX), "fp6_e3m2": (mx.FP6_E3M2_MAGS, mx.FP6_E3M2_QMAX)}


@pytest.mark.parametrize("fmt", FMTS)
def test_grid_extremes_and_ties(fmt):
    mags, qmax = FMTS[fmt]
    g = _read_golden("formats.txt")
    mx_, mn, sub_max, sub_min = (float(v) for v in g[fmt + "_extremes"].split(","))
    assert mags[-1] == mx_ == qmax
    normals = mags[mags >= mn]
    assert mags[1] == sub_min and mags[mags < mn].max() == sub_max and normals.min() == mn
    assert np.all(np.diff(mags) > 0) and len(mags) == 32
    for item in g[fmt + "_ties"].split(";"):
        v, want = (float(a) for a in item.split("->"))
        assert mags[mx.round_to_grid(np.array([v]), mags)[0]] == want, (v, want)


@pytest.mark.parametrize("fmt", FMTS)
def test_element_rounding_brute_force(fmt):
    mags, _ = FMTS[fmt]
    rng = np.random.default_rng(11)
    codes = np.arange(32)
    table_vals = np.concatenate([mags, -mags])
    table_codes = np.concatenate([codes, codes | 32])
    v = _interesting_values(mags, rng, 100_000)
    want = np.empty(len(v), dtype=np.int64)
    for s in range(0, len(v), 4096):
        want[s:s + 4096] = _brute_nearest(v[s:s + 4096], table_vals, table_codes)
    zero = (want & 31) == 0
    want = np.where(zero, np.where(np.signbit(v), 32, 0), want)
    got = mx.round_to_grid(v, mags).astype(np.int64) | np.where(np.signbit(v), 32, 0)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt", FMTS)
def test_scale_exponent_brute_force(fmt):
    _, qmax = FMTS[fmt]
    rng = np.random.default_rng(5)
    a = np.concatenate([rng.uniform(0, 1, 2000) * 2.0 ** rng.integers(-140, 120, 2000),
                        qmax * 2.0 ** np.arange(-130, 120, dtype=np.float64),
                        np.nextafter(np.float32(qmax) * np.float32(2.0) ** np.arange(-120, 100), np.float32(np.inf)),
                        [0.0, 1e-45, 2.0 ** -126, 3.4e38]]).astype(np.float32).astype(np.float64)
    want = np.array([_brute_exponent(x, qmax) for x in a])
    assert np.array_equal(mx.mx_exponent(a, qmax), want)


def test_pack_bit_order():
    # codes 1, 2, 3, 4 -> 1 | 2 << 6 | 3 << 12 | 4 << 18 = 0x103081, little-endian bytes
    assert list(mx.pack_fp6(np.array([[1, 2, 3, 4]], np.uint8))[0]) == [0x81, 0x30, 0x10]
    assert list(mx.pack_fp6(np.array([[63, 0, 0, 0]], np.uint8))[0]) == [0x3F, 0, 0]
    assert list(mx.pack_fp6(np.array([[0, 0, 0, 63]], np.uint8))[0]) == [0, 0, 0xFC]
    c = np.random.default_rng(1).integers(0, 64, (5, 96)).astype(np.uint8)
    assert np.array_equal(mx.unpack_fp6(mx.pack_fp6(c)), c)


@pytest.mark.parametrize("fmt", FMTS)
def test_lossless_on_representable_groups(fmt):
    """Values that are grid points times the group's own scale (the group
    maximum on q_max 2^e) come back unchanged."""
    mags, qmax = FMTS[fmt]
    rng = np.random.default_rng(2)
    e = rng.integers(-20, 20, (16, 4))
    vals = mags[rng.integers(0, 32, (16, 4, 32))] * np.where(rng.random((16, 4, 32)) < 0.5, -1, 1)
    vals[..., 0] = qmax
    x = (vals * np.ldexp(1.0, e)[..., None]).reshape(16, 128).astype(np.float32)
    c, s = mx.mx_quantize(x, fmt)
    assert np.array_equal(mx.mx_dequantize(c, s, fmt), x.astype(np.float64))
    assert np.array_equal(s.astype(np.int64) - 127, e)


def _scalar_layer(x, wt, l1, l2, fmt):
    """Plain loops, one token and one output channel at a time: quantize each
    32-channel group (smallest scale by search, nearest grid value by search,
    ties to even), dot products in Python floats, plus U L2."""
    mags, qmax = FMTS[fmt]
    grid = list(mags)

    def q_group(v):
        amax = max(abs(t) for t in v)
        e = -127
        while e < 127 and amax > qmax * 2.0 ** e:
            e += 1
        out = []
        for t in v:
            a = abs(t) / 2.0 ** e
            best = min(range(32), key=lambda c: (abs(a - grid[c]), c % 2))
            out.append(math.copysign(grid[best], t) * 2.0 ** e)
        return out

    def q_row(row):
        return [y for g in range(len(row) // 32) for y in q_group(row[32 * g:32 * g + 32])]

    r = lowrank.residual(wt, l1, l2)
    rq = [q_row([float(t) for t in row]) for row in r]
    l1f, l2f = mx.bf16_bits_to_f64(l1), mx.bf16_bits_to_f64(l2)
    out = np.zeros((x.shape[0], wt.shape[0]))
    for n in range(x.shape[0]):
        xq = q_row([float(t) for t in x[n]])
        xb = mx.bf16_bits_to_f64(mx.f32_to_bf16_bits(x[n]))
        u = [sum(xb[c] * l1f[c, q] for c in range(x.shape[1])) for q in range(l1.shape[1])]
        u = mx.bf16_bits_to_f64(mx.f64_to_bf16_bits(np.array(u)))
        for j in range(wt.shape[0]):
            out[n, j] = sum(xq[c] * rq[j][c] for c in range(x.shape[1])) + sum(u[q] * l2f[q, j] for q in range(len(u)))
    return out


@pytest.mark.parametrize("fmt", FMTS)
def test_scalar_rederivation_tiny_layer(fmt):
    rng = np.random.default_rng(4)
    N, Ci, Co, r = 6, 64, 12, 4
    x = (rng.standard_normal((N, Ci)) * np.where(rng.random(Ci) < 0.1, 30, 1)).astype(np.float32)
    wt = (rng.standard_normal((Co, Ci)) / 8).astype(np.float32)
    l1, l2, _ = lowrank.svd_factors(wt, r)
    q = text_layer.quantize_text_activation(x, l1, fmt)
    rc, rs = lowrank.quantize_residual(lowrank.residual(wt, l1, l2), fmt)
    y = text_layer.forward(q, rc, rs, l2).astype(np.float64)
    ref = _scalar_layer(x, wt, l1, l2, fmt)
    assert np.all(np.abs(y - ref) <= 2.0 ** -23 * np.abs(ref) + 1e-30)


def test_six_bit_error_below_four_bit():
    """Sanity (not a pin of the pages' numbers): on the same weight and
    activations, W6A6 (either format) has a lower output error than direct
    W4A4 with the same low-rank branch."""
    rng = np.random.default_rng(9)
    N, Ci, Co, r = 64, 256, 96, 16
    x = (rng.standard_normal((N, Ci)) * np.where(rng.random(Ci) < 0.05, 20, 1)).astype(np.float32)
    wt = (rng.standard_normal((Co, Ci)) / 16).astype(np.float32)
    l1, l2, _ = lowrank.svd_factors(wt, r)
    res = lowrank.residual(wt, l1, l2)
    exact = layer.exact_output(x, wt)
    q4 = layer.direct_output(x, layer.low_rank_down(x, l1), l2, *lowrank.quantize_residual(res))
    e4 = layer.rel_fro(q4, exact)
    for fmt in FMTS:
        q = text_layer.quantize_text_activation(x, l1, fmt)
        e6 = layer.rel_fro(text_layer.forward(q, *lowrank.quantize_residual(res, fmt), l2), exact)
        assert e6 < e4, (fmt, e6, e4)
