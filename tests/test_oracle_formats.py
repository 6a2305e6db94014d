"""Pins of the oracle's number formats against things other than itself:
brute-force nearest-code search, torch's own float8_e4m3fn / bfloat16
conversions, brute-force scale search, and the textbook E2M1 value grid."""
import os

import numpy as np
import pytest
import torch

from oracle import mx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    return vals


def test_fp4_grid_matches_textbook_and_page_qmax():
    g = _read_golden("formats.txt")
    grid = [float(v) for v in g["fp4_e2m1_magnitudes"].split(",")]
    assert list(mx.FP4_MAGS) == grid
    # the pages fix q_max = 6 for 4-bit floats: the largest FP4 magnitude
    assert mx.FP4_MAGS[-1] == float(_read_golden("pages.txt")["fp4_qmax"]) == mx.FP4_QMAX


def test_fp8_table_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    for c in range(256):
        mag = mx.FP8_MAGS[c & 0x7F] if (c & 0x7F) < 127 else np.nan
        val = -mag if c & 0x80 else mag
        if np.isnan(ref[c]):
            assert (c & 0x7F) == 0x7F
        else:
            assert val == ref[c], c
    assert mx.FP8_MAGS[-1] == mx.FP8_QMAX == float(_read_golden("formats.txt")["fp8_e4m3_max"])


def _brute_nearest(v, table_vals, table_codes):
    """argmin |v - value|, ties to the even code (the code's low bit is the
    mantissa's low bit), sign of v kept for zero results."""
    d = np.abs(v[:, None] - table_vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even = (table_codes[None, :] % 2 == 0) & cand
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    return table_codes[pick]


def _interesting_values(mags, rng, n_random):
    mids = (mags[:-1] + mags[1:]) / 2
    pts = np.concatenate([mags, mids])
    vals = [pts]
    f = pts.astype(np.float32)
    for k in range(1, 6):     # a few ulps either side of every grid point and midpoint
        vals.append(np.nextafter(f, np.float32(np.inf)).astype(np.float64))
        vals.append(np.nextafter(f, np.float32(0)).astype(np.float64))
        f = np.nextafter(f, np.float32(np.inf))
    bf = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    bf = bf[np.isfinite(bf)].astype(np.float64)
    vals.append(bf[np.abs(bf) <= mags[-1]])
    vals.append(rng.uniform(0, mags[-1], n_random).astype(np.float32).astype(np.float64))
    v = np.concatenate(vals)
    v = v[np.abs(v) <= mags[-1]]
    return np.concatenate([v, -v])


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_element_rounding_brute_force(fmt):
    rng = np.random.default_rng(7)
    mags = mx.FP4_MAGS if fmt == "fp4" else mx.FP8_MAGS
    nmag = len(mags)
    sign_bit = 8 if fmt == "fp4" else 0x80
    codes = np.arange(nmag)
    table_vals = np.concatenate([mags, -mags])
    table_codes = np.concatenate([codes, codes | sign_bit])
    v = _interesting_values(mags, rng, 200_000)
    want = np.empty(len(v), dtype=np.int64)
    for s in range(0, len(v), 4096):
        want[s:s + 4096] = _brute_nearest(v[s:s + 4096], table_vals, table_codes)
    # zero results keep the sign of the input
    zero = (want & (sign_bit - 1)) == 0
    want = np.where(zero, np.where(np.signbit(v), sign_bit, 0), want)
    got = mx.round_to_grid(v, mags).astype(np.int64) | np.where(np.signbit(v), sign_bit, 0)
    assert np.array_equal(got, want)


def test_fp8_rounding_matches_torch():
    """torch's float32 -> float8_e4m3fn cast is round-to-nearest-even."""
    bits = np.arange(0, 2**32, 97, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) <= 448)]
    ref = torch.from_numpy(x.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = mx.round_to_grid(x, mx.FP8_MAGS) | (np.signbit(x).astype(np.uint8) << 7)
    assert np.array_equal(got, ref)


def test_midpoint_table_fp4():
    g = _read_golden("formats.txt")
    for item in g["fp4_ties"].split(";"):
        v, want = (float(a) for a in item.split("->"))
        idx = mx.round_to_grid(np.array([v]), mx.FP4_MAGS)[0]
        assert mx.FP4_MAGS[idx] == want, (v, want)


def _brute_exponent(a, qmax):
    for e in range(-127, 128):
        if a <= qmax * 2.0 ** e:
            return e
    return 127


@pytest.mark.parametrize("qmax", [mx.FP4_QMAX, mx.FP8_QMAX])
def test_scale_exponent_brute_force(qmax):
    rng = np.random.default_rng(11)
    edges = []
    for e in range(-130, 128, 3):
        p = np.float32(qmax * 2.0 ** e) if -149 <= e + 3 and qmax * 2.0 ** e < 3.4e38 else None
        if p is not None and np.isfinite(p):
            edges += [p, np.nextafter(p, np.float32(np.inf)), np.nextafter(p, np.float32(0))]
    edges += [np.float32(0), np.float32(1e-45), np.float32(1.1754942e-38), np.float32(1.1754944e-38),
              np.finfo(np.float32).max]
    rnd = (rng.uniform(-140, 127, 3000)).astype(np.float64)
    edges += list((2.0 ** rnd * rng.uniform(1, 2, 3000)).astype(np.float32))
    a = np.array([v for v in edges if np.isfinite(v)], dtype=np.float32)
    got = mx.mx_exponent(a, qmax)
    want = np.array([max(-127, _brute_exponent(float(v), qmax)) for v in a])
    assert np.array_equal(got, want)
    # independent closed form on the bit pattern: amax = m 2^E, q_max = mq 2^Eq
    b = a.view(np.uint32).astype(np.int64)
    E = (b >> 23) - 127
    mant = b & 0x7FFFFF
    mq, Eq = (0x400000, 2) if qmax == 6.0 else (0x600000, 8)
    closed = np.where((b >> 23) == 0, -127, E - Eq + (mant > mq))
    assert np.array_equal(got, np.clip(closed, -127, 127))


def test_mx_quantize_group_scale_and_zero():
    x = np.zeros((2, 64), dtype=np.float32)
    x[0, :32] = np.linspace(-3, 3, 32, dtype=np.float32)
    x[1, 32:] = -0.0
    codes, scales = mx.mx_quantize(x, "fp4")
    # group max 3 = 0.75 * 2^2 -> smallest e with 3 <= 6 * 2^e is e = -1
    assert scales[0, 0] == 127 - 1
    assert scales[0, 1] == 0 and scales[1, 0] == 0 and scales[1, 1] == 0   # all-zero groups -> 2^-127
    assert np.all(codes[1, 32:] == 0x8) and np.all(codes[1, :32] == 0)      # signed zeros kept
    deq = mx.mx_dequantize(codes, scales, "fp4")
    assert np.all(np.abs(deq[0, :32] - x[0, :32]) <= 2.0 ** -1)             # half the top spacing of 2^e * {4, 6}


def test_mx_quantize_scale_group_64():
    """One exponent per 64 channels (the pages' group-64 FP8 core), pinned by
    properties of the definition: the exponent grows with the maximum, so the
    shared scale code is the larger of the two 32-channel codes; the half that
    sets it is coded exactly as with 32-channel groups; every element of the
    other half takes the nearest FP8 value times the shared scale (brute force
    over all 256 codes, ties to the even code); equal halves change nothing."""
    rng = np.random.default_rng(64)
    x = (rng.standard_normal((6, 256)) * np.exp(rng.uniform(-4, 4, (6, 256)))).astype(np.float32)
    x[2, 64:128] *= 1e-3                                  # one half far below its partner
    c32, s32 = mx.mx_quantize(x, "fp8")
    c64, s64 = mx.mx_quantize(x, "fp8", 64)
    pair = np.maximum(s32[:, 0::2], s32[:, 1::2])
    assert np.array_equal(s64[:, 0::2], pair) and np.array_equal(s64[:, 1::2], pair)
    assert np.any(s32 != s64)                             # the case is not degenerate
    vals = np.array([mx.fp8_decode_magnitude(c & 0x7F) * (-1.0 if c & 0x80 else 1.0) for c in range(256)])
    valid = np.isfinite(vals)
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 32):
            blk = slice(32 * b, 32 * b + 32)
            if s64[r, b] == s32[r, b]:
                assert np.array_equal(c64[r, blk], c32[r, blk])
            scale = 2.0 ** (int(s64[r, b]) - 127)
            for i in range(32 * b, 32 * b + 32):
                err = np.where(valid, np.abs(vals * scale - float(x[r, i])), np.inf)
                best = np.flatnonzero(err == err.min())
                assert int(c64[r, i]) in best, (r, i)
                if len(best) > 1:                         # a tie: the even mantissa
                    assert (int(c64[r, i]) & 1) == 0, (r, i)
    same = np.tile(x[:, :32], (1, 2))                     # equal halves
    assert np.array_equal(mx.mx_quantize(same, "fp8", 64)[0], mx.mx_quantize(same, "fp8")[0])
    with pytest.raises(ValueError):
        mx.mx_quantize(x[:, :96], "fp8", 64)


def test_pack_nibble_order():
    codes = np.array([[1, 2, 3, 4, 0xF, 0x8]], dtype=np.uint8)
    assert list(mx.pack_fp4(codes)[0]) == [0x21, 0x43, 0x8F]
    assert np.array_equal(mx.unpack_fp4(mx.pack_fp4(codes)), codes)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(3)
    rnd = (rng.standard_normal(100_000) * 10.0 ** rng.integers(-20, 20, 100_000)).astype(np.float32)
    ties = ((np.arange(1, 60000, dtype=np.uint32) << 16) + 0x8000).view(np.float32)
    x = np.concatenate([rnd, ties])
    x = x[np.isfinite(x) & (np.abs(x) > 1.2e-38) & (np.abs(x) < 3e38)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mx.f32_to_bf16_bits(x), ref)


def test_bf16_rounding_of_subnormals_and_zeros_matches_torch():
    """Every fp32 subnormal pattern of both signs (the bf16 grid there is the
    fixed spacing 2^-133), the signed zeros, and the smallest normals."""
    mags = np.arange(0, 1 << 23, dtype=np.uint32)
    normals = np.arange(0x00800000, 0x00800000 + (1 << 20), dtype=np.uint32)
    bits = np.concatenate([mags, mags | 0x80000000, normals, normals | 0x80000000])
    x = bits.view(np.float32)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mx.f32_to_bf16_bits(x), ref)
