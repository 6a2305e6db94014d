"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: delta/core/R codes and scale codes bit-exact; U within one bf16 ulp;
the fp32 output within 2e-3 relative Frobenius error (and every row within
2e-3 relative, to catch a misplaced row).  Small layers are compared in
full; the full-size layers on sampled whole cubes (partial cubes included).
Factors L1, L2 come from the oracle's LAPACK SVD (small layers) or from a
seeded generator (full-size layers): parity is about computing the layer
for given factors; the library's own SVD is checked by its properties.
"""
import os
import sys

import numpy as np
import pytest
import torch

from oracle import cubes, layer, lowrank, mx
from w4a4_quantized_linear_cube_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dqm(lib):
    from w4a4_quantized_linear_cube_amd import dq
    return dq


def _random_factors(Ci, Co, r, seed):
    """Seeded bf16 factors of realistic magnitude (not an SVD)."""
    if r == 0:
        return np.zeros((Ci, 0), np.uint16), np.zeros((0, Co), np.uint16)
    g = torch.Generator().manual_seed(seed)
    l1 = (torch.randn(Ci, r, generator=g) * 0.05).to(torch.bfloat16)
    l2 = (torch.randn(r, Co, generator=g) * 0.05).to(torch.bfloat16)
    return (l1.view(torch.int16).numpy().view(np.uint16).copy(), l2.view(torch.int16).numpy().view(np.uint16).copy())


def _ulp_bf16(v):
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def _check_u(got_bits, want_bits, x_rows, l1_bits):
    """U = bf16(bf16(x) L1) with fp32 accumulation on the GPU vs fp64 in the
    oracle: they may differ by one bf16 ulp of rounding plus the fp32
    summation error bound (Ci - 1) 2^-24 sum_c |x_c L1_c| (any order)."""
    g = mx.bf16_bits_to_f64(got_bits)
    w = mx.bf16_bits_to_f64(want_bits)
    xb = np.abs(mx.bf16_bits_to_f64(mx.f32_to_bf16_bits(x_rows)))
    absdot = xb @ np.abs(mx.bf16_bits_to_f64(l1_bits))
    bound = _ulp_bf16(np.maximum(np.abs(g), np.abs(w))) + (x_rows.shape[1] - 1) * 2.0 ** -24 * absdot
    bad = np.argwhere(np.abs(g - w) > bound)
    assert len(bad) == 0, f"U outside the fp32-accumulation bound at {bad[:5]}"


# Per-instruction accuracy of the gfx950 scaled MFMA, measured on random
# full-lane data against exact sums: FP4 x FP4 returns the exact 64-term sum
# rounded once (<= 0.5 ulp; two roundings with a nonzero accumulator), while
# FP8 x FP4 keeps about 13 bits internally (worst 2^-12.6 of sum|products|
# per instruction on random codes, 2^-10.5 with mostly subnormal FP8).
MFMA_FP8_REL = 2.0 ** -9


def _abs_bound(q, g, rc, rs, l2_bits, x_rows, l1_bits):
    """Elementwise bound on |y_gpu - y_oracle| from the arithmetic: the delta
    dot product is Ci/64 MFMA blocks of exact sums each rounded (twice) into an
    fp32 accumulator; the core dot product the same plus MFMA_FP8_REL per
    block; the low-rank dot product r/16 bf16 blocks; plus the low-rank term's
    share of the U difference allowed by _check_u.  The final rounding of y is
    added by the caller."""
    Ci = rc.shape[1] * 2
    r = l2_bits.shape[0]
    rdq = np.abs(mx.mx_dequantize(mx.unpack_fp4(rc), rs, "fp4")).T
    core_abs = np.abs(layer.core_values(q))
    delta_abs = np.abs(mx.mx_dequantize(mx.unpack_fp4(q["delta_codes"]), q["delta_scales"], "fp4"))
    rows = q["row_of_cube"][cubes.cube_of_token(g, q["tokens"])]
    blocks = Ci // 64 + 4
    bound = (blocks * 2.0 ** -23) * (delta_abs @ rdq) + (MFMA_FP8_REL + blocks * 2.0 ** -23) * (core_abs @ rdq)[rows]
    if r:
        u = np.abs(mx.bf16_bits_to_f64(q["U"]))
        l2a = np.abs(mx.bf16_bits_to_f64(l2_bits))
        xb = np.abs(mx.bf16_bits_to_f64(mx.f32_to_bf16_bits(x_rows)))
        ub = 2 * _ulp_bf16(u) + (Ci - 1) * 2.0 ** -24 * (xb @ np.abs(mx.bf16_bits_to_f64(l1_bits)))
        bound = bound + ((r // 16 + 4) * 2.0 ** -23) * ((u + ub) @ l2a) + ub @ l2a
    return bound


def _check_y(y, yo, bound=None):
    err = layer.rel_fro(y, yo)
    num = np.linalg.norm(y.astype(np.float64) - yo, axis=1)
    den = np.linalg.norm(yo.astype(np.float64), axis=1) + 1e-30
    row = float((num / den).max())
    assert err <= TOL, f"rel Frobenius error {err}"
    if bound is not None:
        diff = np.abs(y.astype(np.float64) - yo.astype(np.float64))
        lim = bound + 2.0 ** -23 * np.abs(yo.astype(np.float64))
        bad = np.argwhere(diff > lim)
        worst = float((diff / lim).max())
        assert len(bad) == 0, f"{len(bad)} outputs outside the accumulation bound (worst {worst:.2f}x), first {bad[:5]}"
    return err, row


def _layer(dqm, T, H, W, cube, Ci, Co, rank, dtype, xseed, wseed, svd="oracle", n_out=4, w_out=2, core_group=32,
           core_bits=8):
    x = synth.make_activation(T, H, W, Ci, seed=xseed, dtype=dtype, n_outliers=n_out)
    wt = synth.make_weight(Ci, Co, seed=wseed, dtype=dtype, outlier_rows=w_out)
    xf, wf = synth.to_f32_numpy(x), synth.to_f32_numpy(wt)
    if svd == "oracle" and rank > 0:
        l1, l2, _ = lowrank.svd_factors(wf, rank)
    else:
        l1, l2 = _random_factors(Ci, Co, rank, wseed + 1)
    weights = dqm.dq_prepare_weights_lowrank(wt, l1 if rank else None, l2 if rank else None, device=0)
    qa = dqm.dq_qact_create(weights, (T, H, W) + tuple(cube), core_group=core_group, core_bits=core_bits)
    xd = x.to(DEV)
    y = torch.full((T * H * W, Co), float("nan"), dtype=torch.float32, device=DEV)
    dqm.dq_linear(weights, xd, qa, y)
    torch.cuda.synchronize()
    return dict(x=xf, wt=wf, l1=l1, l2=l2, weights=weights, qa=qa, y=y.cpu().numpy(), g=cubes.Geometry(T, H, W, *cube),
                core_group=core_group, core_bits=core_bits)


def _full_compare(dqm, L):
    got = dqm.dq_qact_export(L["qa"])
    q = layer.quantize_activation(L["x"], L["g"], L["l1"] if L["l1"].shape[1] else None,
                                  core_group=L.get("core_group", 32), core_bits=L.get("core_bits", 8))
    assert np.array_equal(got["core_codes"], q["core_codes"]), "core codes"
    if q["core_scales"] is not None:
        assert np.array_equal(got["core_scales"], q["core_scales"]), "core scales"
    assert np.array_equal(got["delta_scales"], q["delta_scales"]), "delta scales"
    assert np.array_equal(got["delta_codes"], q["delta_codes"]), "delta codes"
    r = lowrank.residual(L["wt"], L["l1"], L["l2"])
    rc, rs = lowrank.quantize_residual(r)
    wexp = dqm.dq_weights_export(L["weights"])
    assert np.array_equal(wexp["r"].view(np.uint32), r.view(np.uint32)), "R"
    assert np.array_equal(wexp["rcodes"], rc) and np.array_equal(wexp["rscales"], rs), "Q4(R)"
    if L["l1"].shape[1]:
        _check_u(got["U"], q["U"], L["x"][q["tokens"]], L["l1"])
    else:
        q["U"] = np.zeros((len(q["tokens"]), 0), np.uint16)
    yo = layer.forward(q, L["g"], rc, rs, L["l2"])
    assert not np.isnan(L["y"]).any(), "unwritten outputs"
    bound = _abs_bound(q, L["g"], rc, rs, L["l2"], L["x"][q["tokens"]], L["l1"])
    return _check_y(L["y"], yo, bound)


# ------------------------------------------------------------------ small ----
def test_tiny_config_full(dqm):
    cfg = synth.CONFIGS["tiny"]
    _say("case tiny config")
    x = synth.config_activation(cfg)
    wt = synth.config_weight(cfg)
    xf, wf = synth.to_f32_numpy(x), synth.to_f32_numpy(wt)
    l1, l2, _ = lowrank.svd_factors(wf, cfg.rank)
    weights = dqm.dq_prepare_weights_lowrank(wt, l1, l2)
    qa = dqm.dq_qact_create(weights, (cfg.T, cfg.H, cfg.W) + cfg.cubes[0])
    y = torch.full((cfg.N, cfg.Co), float("nan"), device=DEV)
    dqm.dq_linear(weights, x.to(DEV), qa, y)
    torch.cuda.synchronize()
    L = dict(x=xf, wt=wf, l1=l1, l2=l2, weights=weights, qa=qa, y=y.cpu().numpy(),
             g=cubes.Geometry(cfg.T, cfg.H, cfg.W, *cfg.cubes[0]))
    err, row = _full_compare(dqm, L)
    _say(f"tiny: rel err {err:.2e} worst row {row:.2e}")


EDGE = [
    # T, H, W, cube, Ci, Co, rank, dtype
    (3, 5, 7, (1, 2, 2), 96, 40, 16, "f32"),       # ragged grid, Ci and Co not tile multiples
    (2, 9, 11, (2, 2, 2), 160, 200, 32, "bf16"),   # partial cubes along all axes
    (4, 6, 6, (1, 1, 1), 128, 64, 0, "bf16"),      # 1x1x1 cubes (delta = 0), no low-rank branch
    (3, 7, 9, (1, 3, 3), 64, 96, 16, "bf16"),      # 9-token cubes
    (3, 10, 12, (2, 3, 5), 256, 300, 48, "bf16"),  # 30-token cubes
    (3, 9, 10, (3, 9, 10), 64, 48, 16, "f32"),     # one global cube of 270 tokens (> 64)
    (5, 7, 9, (4, 4, 8), 128, 128, 128, "bf16"),   # 128-token cubes, clipped; rank 128
    (1, 1, 3, (1, 1, 2), 32, 8, 8, "f32"),         # three tokens
    (2, 16, 16, (1, 4, 4), 512, 256, 32, "bf16"),  # 16-token cubes, several tiles in every dim
    (3, 7, 10, (1, 2, 2), 512, 512, 32, "bf16"),   # 4-token cubes, clipped, pad slots, two channel tiles
    (3, 6, 8, (1, 4, 4), 96, 64, 16, "f32"),        # fp32 input, one wave per 16-token cube (clipped), a partial chunk
    (21, 4, 6, (4, 1, 4), 64, 64, 16, "bf16"),     # the pages' small tile t4 h1 w4 on 21 frames
    (21, 4, 16, (4, 2, 8), 64, 64, 16, "bf16"),    # the pages' large tile t4 h2 w8
    (5, 6, 8, (2, 2, 2), 256, 256, 32, "bf16"),    # last frame alone: second frame segment at row 256
    (4, 6, 10, (2, 2, 2), 128, 96, 16, "f32"),     # fp32 input, 8-token cubes (eight lanes per group)
    (9, 8, 16, (4, 2, 4), 256, 512, 32, "bf16"),   # second frame segment after four tiles of 32-token cubes
    (5, 9, 10, (4, 9, 10), 64, 48, 16, "f32"),     # both frame segments with cubes of more than 64 tokens, fp32 input
]


@pytest.mark.parametrize("case", EDGE, ids=[f"{c[0]}x{c[1]}x{c[2]}_c{'x'.join(map(str, c[3]))}_ci{c[4]}_co{c[5]}_r{c[6]}_{c[7]}"
                                            for c in EDGE])
def test_edge_cases(dqm, case):
    T, H, W, cube, Ci, Co, rank, dtype = case
    _say(f"case edge {case}")
    L = _layer(dqm, T, H, W, cube, Ci, Co, rank, dtype, xseed=T * 100 + Ci, wseed=Co + 7,
               n_out=min(4, Ci // 16))
    err, row = _full_compare(dqm, L)
    _say(f"edge {case}: rel err {err:.2e} worst row {row:.2e}")


# group-64 cores (one FP8 exponent per 64 channels), through every form of
# the activation pass: one-pass (4-token cubes), eighths (8), wave per cube
# (16), two phases with channel pairs (32) and single channels (64), the
# partial-sum pass (cubes of more than 64 tokens), one-token cubes
CORE64 = [
    (3, 7, 10, (1, 2, 2), 256, 256, 32, "bf16"),
    (2, 5, 6, (1, 2, 2), 128, 64, 16, "f32"),
    (4, 6, 10, (2, 2, 2), 256, 96, 16, "bf16"),
    (3, 6, 8, (1, 4, 4), 128, 64, 16, "bf16"),
    (3, 8, 8, (2, 4, 4), 128, 64, 16, "bf16"),
    (5, 7, 9, (4, 4, 4), 192, 64, 16, "bf16"),
    (5, 7, 9, (4, 4, 4), 128, 64, 16, "f32"),
    (3, 9, 10, (3, 9, 10), 128, 48, 16, "bf16"),
    (2, 6, 6, (1, 1, 1), 128, 64, 16, "bf16"),
]


@pytest.mark.parametrize("case", CORE64, ids=[f"{c[0]}x{c[1]}x{c[2]}_c{'x'.join(map(str, c[3]))}_ci{c[4]}_{c[7]}"
                                              for c in CORE64])
def test_core_group_64(dqm, case):
    T, H, W, cube, Ci, Co, rank, dtype = case
    _say(f"case core group 64 {case}")
    L = _layer(dqm, T, H, W, cube, Ci, Co, rank, dtype, xseed=T * 100 + Ci + 64, wseed=Co + 9,
               n_out=min(4, Ci // 16), core_group=64)
    err, row = _full_compare(dqm, L)
    _say(f"core group 64 {case}: rel err {err:.2e} worst row {row:.2e}")


# 4-bit cores (the 4-bit point of the pages' core-precision ablation), through
# the same forms; the last case combines them with group-64 scales
@pytest.mark.parametrize("case", CORE64, ids=[f"{c[0]}x{c[1]}x{c[2]}_c{'x'.join(map(str, c[3]))}_ci{c[4]}_{c[7]}"
                                              for c in CORE64])
def test_core_fp4(dqm, case):
    T, H, W, cube, Ci, Co, rank, dtype = case
    _say(f"case fp4 cores {case}")
    L = _layer(dqm, T, H, W, cube, Ci, Co, rank, dtype, xseed=T * 100 + Ci + 4, wseed=Co + 11,
               n_out=min(4, Ci // 16), core_bits=4, core_group=64 if cube == (2, 2, 2) else 32)
    err, row = _full_compare(dqm, L)
    _say(f"fp4 cores {case}: rel err {err:.2e} worst row {row:.2e}")


# bf16 cores (the 16-bit point of the pages' core-precision ablation: the
# cores rounded to bf16, the core term a library bf16 GEMM against Q4(R)),
# through every form of the activation pass
@pytest.mark.parametrize("case", CORE64, ids=[f"{c[0]}x{c[1]}x{c[2]}_c{'x'.join(map(str, c[3]))}_ci{c[4]}_{c[7]}"
                                              for c in CORE64])
def test_core_bf16(dqm, case):
    T, H, W, cube, Ci, Co, rank, dtype = case
    _say(f"case bf16 cores {case}")
    L = _layer(dqm, T, H, W, cube, Ci, Co, rank, dtype, xseed=T * 100 + Ci + 16, wseed=Co + 13,
               n_out=min(4, Ci // 16), core_bits=16)
    err, row = _full_compare(dqm, L)
    _say(f"bf16 cores {case}: rel err {err:.2e} worst row {row:.2e}")


def test_core_group_errors(dqm):
    wt = synth.make_weight(96, 64, seed=3, dtype="f32")
    weights = dqm.dq_prepare_weights_lowrank(wt, None, None)
    with pytest.raises(dqm.DQError, match="DQ_ERR_SHAPE"):
        dqm.dq_qact_create(weights, (2, 2, 2, 1, 1, 1), core_group=64)      # 64 does not divide Ci = 96
    with pytest.raises(dqm.DQError, match="DQ_ERR_INVALID_ARG"):
        dqm.dq_qact_create(weights, (2, 2, 2, 1, 1, 1), core_group=48)
    with pytest.raises(dqm.DQError, match="DQ_ERR_INVALID_ARG"):
        dqm.dq_qact_create(weights, (2, 2, 2, 1, 1, 1), core_bits=6)


def test_wan1p3b_projection_full(dqm):
    cfg = synth.CONFIGS["wan1p3b_proj"]
    _say("case wan1p3b_proj full")
    L = _layer(dqm, cfg.T, cfg.H, cfg.W, cfg.cubes[0], cfg.Ci, cfg.Co, cfg.rank, cfg.dtype,
               cfg.x_seeds[0], cfg.w_seed, svd="oracle", n_out=cfg.n_outliers, w_out=0)
    err, row = _full_compare(dqm, L)
    _say(f"wan1p3b_proj: rel err {err:.2e} worst row {row:.2e}")


def test_two_runs_bit_identical(dqm):
    _say("case determinism")
    T, H, W, Ci, Co = 4, 10, 12, 256, 512
    x = synth.make_activation(T, H, W, Ci, seed=5, dtype="bf16", n_outliers=4).to(DEV)
    wt = synth.make_weight(Ci, Co, seed=6, dtype="bf16")
    l1, l2 = _random_factors(Ci, Co, 32, 9)
    weights = dqm.dq_prepare_weights_lowrank(wt, l1, l2)
    qa = dqm.dq_qact_create(weights, (T, H, W, 1, 2, 2))
    outs = []
    for _ in range(2):
        y = torch.empty(T * H * W, Co, device=DEV)
        dqm.dq_linear(weights, x, qa, y)
        torch.cuda.synchronize()
        outs.append((y.cpu().numpy().view(np.uint32), dqm.dq_qact_export(qa)))
    assert np.array_equal(outs[0][0], outs[1][0])
    for k in outs[0][1]:
        assert np.array_equal(outs[0][1][k], outs[1][1][k]), k



def test_forward_halves_match_forward(dqm):
    """dq_core_term then dq_delta_term is dq_linear_forward (the same launches)."""
    _say("case forward halves")
    T, H, W, Ci, Co = 4, 10, 12, 256, 512
    x = synth.make_activation(T, H, W, Ci, seed=15, dtype="bf16", n_outliers=4).to(DEV)
    wt = synth.make_weight(Ci, Co, seed=16, dtype="bf16")
    l1, l2 = _random_factors(Ci, Co, 32, 19)
    weights = dqm.dq_prepare_weights_lowrank(wt, l1, l2)
    qa = dqm.dq_qact_create(weights, (T, H, W, 1, 2, 2))
    dqm.dq_quantize_act(weights, x, qa)
    y1 = torch.full((T * H * W, Co), float("nan"), device=DEV)
    y2 = torch.full((T * H * W, Co), float("nan"), device=DEV)
    dqm.dq_linear_forward(weights, qa, y1)
    dqm.dq_core_term(weights, qa)
    dqm.dq_delta_term(weights, qa, y2)
    torch.cuda.synchronize()
    assert np.array_equal(y1.cpu().numpy().view(np.uint32), y2.cpu().numpy().view(np.uint32))

def test_library_svd_path(dqm):
    """dq_prepare_weights: the host SVD factors meet Eckart-Young, and R / Q4(R)
    follow from them (R = fl32(W - L1 L2) within one rounding; codes decode to
    within the MX-FP4 step of R)."""
    _say("case library svd")
    Ci, Co, r = 256, 384, 32
    wt = synth.make_weight(Ci, Co, seed=31, dtype="bf16", outlier_rows=3)
    weights = dqm.dq_prepare_weights(wt, r, seed=3)
    e = dqm.dq_weights_export(weights)
    wf = synth.to_f32_numpy(wt)
    s = np.linalg.svd(wf.astype(np.float64), compute_uv=False)
    ey = lowrank.eckart_young_ratio(wf, e["l1"], e["l2"], s)
    assert ey["err"] <= (1 + 1e-3) * ey["best"] + ey["bf16_slack"], ey
    p = (mx.bf16_bits_to_f64(e["l1"]) @ mx.bf16_bits_to_f64(e["l2"])).T
    exact = wf.astype(np.float64) - p
    assert np.all(np.abs(e["r"] - exact) <= 2.0 ** -24 * np.abs(exact))
    deq = mx.mx_dequantize(mx.unpack_fp4(e["rcodes"]), e["rscales"], "fp4")
    step = np.ldexp(1.0, e["rscales"].astype(np.int64) - 127)          # 2^e: half the widest FP4 gap
    assert np.all(np.abs(deq - e["r"]).reshape(Co, Ci // 32, 32) <= step[..., None])


# -------------------------------------------------------- full size, sampled ----
def _sample_cubes(g, n, seed):
    rng = np.random.default_rng(seed)
    tbl, cnt = cubes.cube_tokens(g)
    partial = np.nonzero(cnt < g.S)[0]
    full = np.nonzero(cnt == g.S)[0]
    pick = list(rng.choice(full, size=min(n, len(full)), replace=False))
    if len(partial):
        pick += list(rng.choice(partial, size=min(8, len(partial)), replace=False))
    pick += [0, g.K - 1]
    return np.unique(np.array(pick, dtype=np.int64))


_WEIGHT_CACHE = {}


def _oracle_weight(cfg):
    """W, seeded factors, and the oracle's R and Q4(R) for a config (cached)."""
    if cfg.name not in _WEIGHT_CACHE:
        wt = synth.config_weight(cfg)
        l1, l2 = _random_factors(cfg.Ci, cfg.Co, cfg.rank, cfg.w_seed + 1)
        wf = synth.to_f32_numpy(wt)
        r = lowrank.residual(wf, l1, l2)
        rc, rs = lowrank.quantize_residual(r)
        _WEIGHT_CACHE.clear()
        _WEIGHT_CACHE[cfg.name] = (wt, l1, l2, r, rc, rs)
    return _WEIGHT_CACHE[cfg.name]


def _full_size_case(dqm, cfg, cube, xseed, check_weights, n_cubes=48, max_rows=512, versus_direct=False):
    T, H, W = cfg.T, cfg.H, cfg.W
    g = cubes.Geometry(T, H, W, *cube)
    _say(f"case {cfg.name} cube {cube} seed {xseed}: generating")
    x = synth.make_activation(T, H, W, cfg.Ci, seed=xseed, dtype=cfg.dtype, n_outliers=cfg.n_outliers, device=DEV)
    wt, l1, l2, r, rc, rs = _oracle_weight(cfg)
    weights = dqm.dq_prepare_weights_lowrank(wt, l1, l2)
    qa = dqm.dq_qact_create(weights, (T, H, W) + tuple(cube))
    y = torch.full((cfg.N, cfg.Co), float("nan"), device=DEV)
    _say(f"case {cfg.name} cube {cube}: running")
    dqm.dq_linear(weights, x, qa, y)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any().item(), "unwritten outputs"
    got = dqm.dq_qact_export(qa)
    ids = _sample_cubes(g, n_cubes, xseed)
    tbl, cnt = cubes.cube_tokens(g, ids)
    toks = np.sort(tbl[tbl >= 0])
    rng = np.random.default_rng(xseed)
    if len(toks) > max_rows:          # keep every partial cube's tokens, sample the rest
        part = np.isin(cubes.cube_of_token(g, toks), ids[cnt < g.S])
        keep = np.concatenate([toks[part][:max_rows // 2],
                               rng.choice(toks[~part], size=max_rows - min(part.sum(), max_rows // 2), replace=False)])
        toks = np.sort(keep)
    xf = synth.to_f32_numpy(x)
    _say(f"case {cfg.name} cube {cube}: oracle on {len(ids)} cubes, {len(toks)} tokens")
    q = layer.quantize_activation(xf, g, l1, cube_ids=ids, tokens=toks)
    assert np.array_equal(got["core_codes"][ids], q["core_codes"]), "core codes"
    assert np.array_equal(got["core_scales"][ids], q["core_scales"]), "core scales"
    assert np.array_equal(got["delta_codes"][q["tokens"]], q["delta_codes"]), "delta codes"
    assert np.array_equal(got["delta_scales"][q["tokens"]], q["delta_scales"]), "delta scales"
    _check_u(got["U"][q["tokens"]], q["U"], xf[q["tokens"]], l1)
    if check_weights:
        e = dqm.dq_weights_export(weights)
        assert np.array_equal(e["r"].view(np.uint32), r.view(np.uint32)), "R"
        assert np.array_equal(e["rcodes"], rc) and np.array_equal(e["rscales"], rs), "Q4(R)"
    yo = layer.forward(q, g, rc, rs, l2)
    bound = _abs_bound(q, g, rc, rs, l2, xf[q["tokens"]], l1)
    err, row = _check_y(y.cpu().numpy()[q["tokens"]], yo, bound)
    _say(f"{cfg.name} cube {cube} seed {xseed}: codes bit-exact on {len(ids)} cubes; "
         f"Y rel err {err:.2e} worst row {row:.2e} on {len(q['tokens'])} tokens")
    if versus_direct:
        # output error against the exact X W (fp64) on 128 of the sampled
        # tokens: delta W4A4 (the GPU output) and direct W4A4 of X (oracle:
        # the same R, rank and MX rule, X quantized per token without a core)
        t = q["tokens"][:128]
        ex = layer.exact_output(xf[t], synth.to_f32_numpy(wt))
        e_dq = layer.rel_fro(y.cpu().numpy()[t], ex)
        e_dir = layer.rel_fro(layer.direct_output(xf[t], q["U"][:128], l2, rc, rs), ex)
        _say(f"{cfg.name} cube {cube}: error vs exact X W on {len(t)} tokens: delta W4A4 {e_dq:.3e}, "
             f"direct W4A4 {e_dir:.3e} (ratio {e_dq / e_dir:.3f})")
        # the core removes shared content before the 4-bit step (关键设计 3):
        # never worse than direct W4A4 beyond noise (a single global cube is
        # the degenerate case, about equal)
        assert e_dq <= 1.02 * e_dir, (e_dq, e_dir)


def test_attn14b_projection_sampled(dqm):
    cfg = synth.CONFIGS["attn14b_proj"]
    for i, seed in enumerate(cfg.x_seeds):          # the outlier set is redrawn per timestep seed
        _full_size_case(dqm, cfg, cfg.cubes[0], seed, check_weights=(i == 0), n_cubes=24)


def test_ffn_up_720p_sampled(dqm):
    cfg = synth.CONFIGS["ffn_up_720p"]
    _full_size_case(dqm, cfg, cfg.cubes[0], cfg.x_seeds[0], check_weights=True)


@pytest.mark.parametrize("cube,step", [((4, 1, 4), 0), ((4, 2, 8), 1)], ids=["4x1x4", "4x2x8"])
def test_ffn_up_720p_schedule_shapes(dqm, cube, step):
    """The timestep-aware cube sizes (DeltaQuant notes, 损失函数/训练策略) at
    full size: 16-token cubes early in denoising (one quantizer wave per cube),
    64-token cubes later (the two-phase quantizer), each on its own synthetic
    timestep's activations; codes bit-exact on sampled cubes, Y within the
    bound, and delta W4A4 no worse than direct W4A4."""
    cfg = synth.CONFIGS["ffn_up_720p"]
    _full_size_case(dqm, cfg, cube, cfg.x_seeds[0] + step, check_weights=False, n_cubes=24 // (1 + step),
                    versus_direct=True)


@pytest.mark.parametrize("cube", synth.CONFIGS["ffn_down_720p"].cubes, ids=lambda c: "x".join(map(str, c)))
def test_ffn_down_720p_sampled(dqm, cube):
    cfg = synth.CONFIGS["ffn_down_720p"]
    _full_size_case(dqm, cfg, cube, cfg.x_seeds[0], check_weights=(cube == (1, 2, 2)), n_cubes=24, versus_direct=True)
