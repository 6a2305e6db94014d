"""Pins of the OrbitQuant-style front end of the oracle (the OrbitQuant page:
RPBH rotation, Lloyd-Max codebook): Max's published Gaussian quantizers and
their distortions, the optimality conditions by numerical integration, the
block Hadamard against the explicit Sylvester matrix, the rotation cancelling
in a product, the tie rule of the nearest level, the RMS order by a scalar
re-derivation, and a scalar re-derivation of a tiny layer."""
import math

import numpy as np
import pytest
from scipy import integrate, linalg, stats

from oracle import mx, orbit
from test_oracle_formats import _read_golden


@pytest.mark.parametrize("L", [2, 4, 8, 16])
def test_lloyd_max_matches_max_1960(L):
    g = _read_golden("lloyd_max.txt")
    want = np.array([float(v) for v in g[f"levels_{L}"].split(",")])
    y = orbit.lloyd_max_gaussian(L)
    assert np.allclose(y, -y[::-1], atol=1e-12)                       # symmetric
    assert np.all(np.abs(y[L // 2:] - want) <= 6e-4), (y[L // 2:], want)
    t = np.concatenate([[-np.inf], (y[:-1] + y[1:]) / 2, [np.inf]])
    mse = sum(integrate.quad(lambda x, yi=yi: (x - yi) ** 2 * stats.norm.pdf(x), t[i], t[i + 1])[0]
              for i, yi in enumerate(y))
    assert abs(mse - float(g[f"mse_{L}"])) <= 2e-3 * float(g[f"mse_{L}"])


@pytest.mark.parametrize("L", [4, 16])
def test_lloyd_max_optimality_conditions(L):
    """Each level is the conditional mean of its cell (integrated numerically
    with scipy, independent of the closed form the oracle iterates)."""
    y = orbit.lloyd_max_gaussian(L)
    t = np.concatenate([[-np.inf], (y[:-1] + y[1:]) / 2, [np.inf]])
    for i in range(L):
        m = integrate.quad(lambda x: x * stats.norm.pdf(x), t[i], t[i + 1])[0]
        p = stats.norm.cdf(t[i + 1]) - stats.norm.cdf(t[i])
        assert abs(m / p - y[i]) < 1e-9


def test_block_hadamard_is_sylvester_matrix():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 512)).astype(np.float32)
    H = linalg.hadamard(256) / 16.0
    want = np.concatenate([x[:, :256].astype(np.float64) @ H.T, x[:, 256:].astype(np.float64) @ H.T], axis=1)
    got = orbit.fwht_blocks(x)
    assert np.max(np.abs(got - want)) <= 1e-5 * np.max(np.abs(want))
    # orthonormal and symmetric: applying it twice gives x back (up to rounding); norms kept
    assert np.allclose(orbit.fwht_blocks(got), x, rtol=1e-5, atol=1e-5)
    assert np.allclose(np.linalg.norm(got, axis=1), np.linalg.norm(x, axis=1), rtol=1e-5)
    with pytest.raises(ValueError):
        orbit.fwht_blocks(x, 128)                                     # not a power of four


def test_rotation_cancels_in_the_product():
    """(x R^T)(w R^T)^T = x w^T: the weight absorbs the rotation offline."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 512)).astype(np.float32)
    w = rng.standard_normal((9, 512)).astype(np.float32)
    perm = rng.permutation(512)
    xr = orbit.rpbh(x, perm).astype(np.float64)
    wr = orbit.rpbh(w, perm).astype(np.float64)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.max(np.abs(xr @ wr.T - ref)) <= 1e-4 * np.max(np.abs(ref))
    # the permutation matters: without it the rotated products differ from x w^T rotated by another perm
    assert not np.allclose(orbit.rpbh(x, perm), orbit.rpbh(x, np.arange(512)))


def test_nearest_level_brute_force_and_ties():
    cb = orbit.codebook_bf16(4)
    lv = mx.bf16_bits_to_f64(cb)
    rng = np.random.default_rng(3)
    mids = (lv[:-1] + lv[1:]) / 2
    v = np.concatenate([rng.standard_normal(20000) * 1.5, mids, lv, [0.0, -0.0, 10.0, -10.0]]).astype(np.float32)
    got = orbit.nearest_level(v, cb)
    for x, c in zip(v.astype(np.float64), got):
        d = np.abs(x - lv)
        best = np.flatnonzero(d == d.min())
        assert c == (best[best % 2 == 0][0] if np.any(best % 2 == 0) else best[0])
    # a midpoint goes to the even index
    assert all(orbit.nearest_level(np.array([m], np.float32), cb)[0] % 2 == 0 for m in mids.astype(np.float32)
               if float(np.float32(m)) == m)


def test_rms_scale_order_scalar_rederivation():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((3, 768)) * np.exp(rng.standard_normal(768))).astype(np.float32)
    got = orbit.rms_scale(x)
    for r in range(3):
        tot = None
        for blk in range(3):
            part = None
            for i in range(256):
                v = x[r, 256 * blk + i]
                sq = np.float32(v * v)
                part = sq if part is None else np.float32(part + sq)
            tot = part if tot is None else np.float32(tot + part)
        assert got[r] == np.float32(np.sqrt(np.float32(tot / np.float32(768))))
    assert np.allclose(got, np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=1)), rtol=1e-5)


def test_tiny_layer_scalar_rederivation():
    """Rotation by the explicit matrix in fp64, normalization, nearest level
    and the scaled sum, one element at a time, against the oracle's layer."""
    rng = np.random.default_rng(5)
    N, Co, C = 4, 6, 256
    x = rng.standard_normal((N, C)).astype(np.float32)
    w = (rng.standard_normal((Co, C)) / 16).astype(np.float32)
    perm = rng.permutation(C)
    cb = orbit.codebook_bf16(4)
    qx, qw = orbit.quantize_rows(x, perm, cb), orbit.quantize_rows(w, perm, cb)
    y = orbit.forward(qx, qw, cb, cb)
    H = linalg.hadamard(C) / 16.0
    lv = mx.bf16_bits_to_f64(cb)
    for n in range(N):
        xr = H @ x[n, perm].astype(np.float64)
        sx = math.sqrt(float(np.sum(xr ** 2)) / C)
        for j in range(Co):
            wr = H @ w[j, perm].astype(np.float64)
            sw = math.sqrt(float(np.sum(wr ** 2)) / C)
            acc = sum(lv[np.argmin(np.abs(a / sx - lv))] * lv[np.argmin(np.abs(b / sw - lv))] for a, b in zip(xr, wr))
            assert abs(y[n, j] - acc * sx * sw) <= 1e-3 * abs(acc * sx * sw) + 1e-6


def test_rotation_spreads_outliers():
    """Sanity of the method's premise: after the rotation a channel outlier
    no longer dominates its block, and the codebook's error is near Max's
    distortion (the rotated coordinates are close to N(0, 1))."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 1024)).astype(np.float32)
    x[:, 17] *= 80.0
    perm = rng.permutation(1024)
    q = orbit.quantize_rows(x, perm, orbit.codebook_bf16(4))
    v = q["rot"] / q["scale"][:, None]
    assert np.max(np.abs(v)) < 6 and np.max(np.abs(x / np.sqrt(np.mean(x ** 2, axis=1, keepdims=True)))) > 20
    lv = mx.bf16_bits_to_f64(orbit.codebook_bf16(4))
    y = rng.standard_normal(200000)
    mse = np.mean((y - lv[orbit.nearest_level(y.astype(np.float32), orbit.codebook_bf16(4))]) ** 2)
    assert abs(mse - 0.009497) < 0.0005
