"""Pins of the oracle's cube partition, core and delta (关键设计 2 and 3):
brute-force enumeration, exact dyadic invariants, the 1x1x1 and global-cube
degenerate cases, and a scalar re-derivation of the blocked fp32 sum."""
import itertools
import os

import numpy as np
import pytest
import torch

from oracle import cubes, mx
from w4a4_quantized_linear_cube_amd import synth

GEOMS = [(4, 8, 8, 1, 2, 2), (3, 5, 7, 2, 2, 3), (21, 45, 6, 1, 2, 2), (5, 3, 4, 4, 1, 4),
         (2, 3, 3, 2, 3, 3), (3, 4, 5, 1, 1, 1), (3, 4, 5, 3, 4, 5)]


@pytest.mark.parametrize("geom", GEOMS)
def test_cube_membership_brute_force(geom):
    g = cubes.Geometry(*geom)
    T, H, W, t, h, w = geom
    members = {}
    for ti, hi, wi in itertools.product(range(T), range(H), range(W)):   # lexicographic token order
        key = (ti // t, hi // h, wi // w)
        members.setdefault(key, []).append((ti * H + hi) * W + wi)
    Tc, Hc, Wc = -(-T // t), -(-H // h), -(-W // w)
    assert g.K == Tc * Hc * Wc == len(members)
    tbl, cnt = cubes.cube_tokens(g)
    k_of = cubes.cube_of_token(g)
    for (a, b, c), toks in members.items():
        k = (a * Hc + b) * Wc + c
        assert cnt[k] == len(toks)
        # within a cube, tokens in lexicographic (dt, dh, dw) order = ascending (t, h, w) order
        assert list(tbl[k, :cnt[k]]) == sorted(toks, key=lambda n: (n // (H * W), (n // W) % H, n % W))
        assert np.all(tbl[k, cnt[k]:] == -1)
        assert np.all(k_of[toks] == k)


def test_page_tile_sizes():
    path = os.path.join(os.path.dirname(__file__), "golden", "pages.txt")
    vals = {k.strip(): v.strip() for k, v in (l.split("=", 1) for l in open(path) if "=" in l and not l.startswith("#"))}
    for key in ("small_tile", "large_tile"):
        t, h, w, s = (int(v) for v in vals[key].strip().split(","))
        g = cubes.Geometry(21, 45, 80, t, h, w)
        assert g.S == s
        _, cnt = cubes.cube_tokens(g)
        assert cnt.sum() == g.N        # every token in exactly one cube, partial cubes included


@pytest.mark.parametrize("geom", [(4, 8, 8, 1, 2, 2), (4, 4, 4, 2, 2, 2), (2, 8, 16, 1, 4, 4), (4, 8, 8, 4, 8, 8)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dyadic_exact_reconstruction(geom, dtype):
    """With x = k 2^-8 and power-of-two counts every sum, mean and delta is
    exact, so core + delta == x bit for bit and the deltas of a cube sum to 0."""
    g = cubes.Geometry(*geom)
    kmax = 2 ** 12 if dtype == "f32" else 2 ** 8
    x = synth.to_f32_numpy(synth.dyadic_activation(g.N, 64, seed=5, kmax=kmax, dtype=dtype))
    core = cubes.cube_core(x, g)
    tbl, cnt = cubes.cube_tokens(g)
    assert set(cnt) == {g.S}
    exact_mean = np.stack([x[tbl[k]].astype(np.float64).mean(axis=0) for k in range(g.K)])
    assert np.array_equal(core.astype(np.float64), exact_mean)
    d = cubes.cube_delta(x, core, g, np.arange(g.N))
    k_of = cubes.cube_of_token(g)
    assert np.array_equal((core[k_of] + d).astype(np.float32), x)
    sums = np.zeros((g.K, 64))
    np.add.at(sums, k_of, d.astype(np.float64))
    assert np.all(sums == 0)


@pytest.mark.parametrize("geom", [(3, 5, 7, 2, 2, 3), (4, 8, 8, 1, 2, 2), (2, 9, 9, 2, 9, 9)])
def test_general_inputs_error_bounds(geom):
    g = cubes.Geometry(*geom)
    x = synth.to_f32_numpy(synth.make_activation(g.T, g.H, g.W, 64, seed=9, dtype="f32", n_outliers=4))
    core = cubes.cube_core(x, g)
    d = cubes.cube_delta(x, core, g, np.arange(g.N))
    k_of = cubes.cube_of_token(g)
    x64, c64, d64 = x.astype(np.float64), core[k_of].astype(np.float64), d.astype(np.float64)
    # delta is x - core rounded once: |core + delta - x| <= 2^-24 |x - core|
    assert np.all(np.abs(c64 + d64 - x64) <= 2.0 ** -24 * np.abs(x64 - c64))
    # core vs the fp64 mean: sequential fp32 sum error + one division rounding
    tbl, cnt = cubes.cube_tokens(g)
    for k in range(g.K):
        xs = x64[tbl[k, :cnt[k]]]
        mean = xs.mean(axis=0)
        bound = (cnt[k] + 1) * 2.0 ** -24 * np.abs(xs).sum(axis=0) / cnt[k] + 2.0 ** -24 * np.abs(mean)
        assert np.all(np.abs(core[k] - mean) <= bound)


def test_unit_cube_gives_zero_delta():
    g = cubes.Geometry(3, 4, 5, 1, 1, 1)
    x = synth.to_f32_numpy(synth.make_activation(3, 4, 5, 64, seed=2, dtype="bf16", n_outliers=3))
    x[0, :5] = -0.0
    core = cubes.cube_core(x, g)
    assert np.array_equal(core.view(np.uint32), x.view(np.uint32))      # the mean of one token is the token
    d = cubes.cube_delta(x, core, g, np.arange(g.N))
    assert np.all(d.view(np.uint32) == 0)                               # +0 everywhere
    codes, scales = mx.mx_quantize(d, "fp4")
    assert np.all(codes == 0) and np.all(scales == 0)


def test_global_cube_is_column_mean():
    """One cube over every token: a single core equal to the column mean
    (the global-core degenerate case of 关键设计 2), shared by all tokens."""
    T, H, W = 3, 9, 10          # 270 tokens: five 64-blocks, the last one partial
    g = cubes.Geometry(T, H, W, T, H, W)
    x = synth.to_f32_numpy(synth.make_activation(T, H, W, 32, seed=4, dtype="f32", n_outliers=2))
    core = cubes.cube_core(x, g)
    assert core.shape == (1, 32)
    x64 = x.astype(np.float64)
    mean = x64.mean(axis=0)
    n = g.N
    bound = (64 + 5) * 2.0 ** -24 * np.abs(x64).sum(axis=0) / n + 2.0 ** -24 * np.abs(mean)
    assert np.all(np.abs(core[0] - mean) <= bound)
    assert np.all(cubes.cube_of_token(g) == 0)


def _scalar_blocked_mean(rows):
    """Independent scalar re-derivation of reading R3 with numpy fp32 scalars."""
    blocks = [rows[i:i + 64] for i in range(0, len(rows), 64)]
    partials = []
    for blk in blocks:
        s = np.float32(blk[0])
        for v in blk[1:]:
            s = np.float32(s + np.float32(v))
        partials.append(s)
    tot = partials[0]
    for p in partials[1:]:
        tot = np.float32(tot + p)
    return np.float32(tot / np.float32(len(rows)))


def test_blocked_sum_order_scalar():
    rng = np.random.default_rng(1)
    g = cubes.Geometry(2, 10, 13, 2, 10, 13)          # one cube of 260 tokens
    x = (rng.standard_normal((g.N, 3)) * np.array([1.0, 1e3, 1e-3])).astype(np.float32)
    x[::7, 0] *= 1e4                                  # large dynamic range: order matters
    core = cubes.cube_core(x, g)
    for c in range(3):
        assert core[0, c] == _scalar_blocked_mean(list(x[:, c]))
    # partial cubes of several sizes against the same scalar rule
    g2 = cubes.Geometry(5, 7, 9, 2, 3, 4)
    x2 = rng.standard_normal((g2.N, 2)).astype(np.float32) * 100
    core2 = cubes.cube_core(x2, g2)
    tbl, cnt = cubes.cube_tokens(g2)
    for k in range(g2.K):
        for c in range(2):
            assert core2[k, c] == _scalar_blocked_mean(list(x2[tbl[k, :cnt[k]], c]))


def test_negative_zero_cube_core():
    g = cubes.Geometry(1, 2, 2, 1, 2, 2)
    x = np.full((4, 32), -0.0, dtype=np.float32)
    core = cubes.cube_core(x, g)
    assert np.all(np.signbit(core))          # the sum starts from the first token, not from +0


def test_subset_matches_full():
    g = cubes.Geometry(4, 9, 7, 2, 2, 2)
    x = synth.to_f32_numpy(synth.make_activation(4, 9, 7, 64, seed=8, dtype="bf16", n_outliers=2))
    full = cubes.cube_core(x, g)
    ids = np.array([0, 5, g.K - 1, 11])
    assert np.array_equal(cubes.cube_core(x, g, ids), full[ids])


def test_generator_deterministic_and_shaped():
    a = synth.make_activation(3, 4, 5, 64, seed=12, dtype="bf16", n_outliers=4)
    b = synth.make_activation(3, 4, 5, 64, seed=12, dtype="bf16", n_outliers=4)
    assert a.dtype == torch.bfloat16 and a.shape == (60, 64)
    assert torch.equal(a, b)
    c = synth.make_activation(3, 4, 5, 64, seed=13, dtype="bf16", n_outliers=4)
    assert not torch.equal(a, c)
    w = synth.make_weight(64, 48, seed=3, dtype="f32", outlier_rows=2, outlier_factor=10.0)
    assert w.shape == (48, 64)
    norms = w.norm(dim=1)
    assert (norms > 5 * norms.median()).sum() == 2
