"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: delta/core/R codes and scale codes bit-exact; U within one bf16 ulp
plus the fp32 summation bound; the fp32 output within 2e-3 relative
Frobenius error, every element inside the accumulation bound derived from
the instruction precisions (_abs_bound), and every row within ROW_TOL
relative (a misplaced or wrong row is off by O(1)).  Single rows can exceed
2e-3 relative where their terms cancel: the FP8 x FP4 MFMA keeps about 13
bits, and the worst row measured is 3.5e-3 (720p FFN down, 1x4x4 cubes).
Small layers are compared in full; the full-size layers' codes and scales on
every cube, their outputs on sampled whole cubes (partial cubes included).
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
from parity_util import (DEV, ROW_TOL, TOL, _abs_bound, _check_u, _check_y, _full_compare, _layer, _random_factors,
                         _say)
from w4a4_quantized_linear_cube_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dqm(lib):
    from w4a4_quantized_linear_cube_amd import dq
    return dq


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
# cores rounded to bf16, the core term a bf16 MFMA GEMM against Q4(R) decoded
# to bf16), through every form of the activation pass
@pytest.mark.parametrize("case", CORE64, ids=[f"{c[0]}x{c[1]}x{c[2]}_c{'x'.join(map(str, c[3]))}_ci{c[4]}_{c[7]}"
                                              for c in CORE64])
def test_core_bf16(dqm, case):
    T, H, W, cube, Ci, Co, rank, dtype = case
    _say(f"case bf16 cores {case}")
    L = _layer(dqm, T, H, W, cube, Ci, Co, rank, dtype, xseed=T * 100 + Ci + 16, wseed=Co + 13,
               n_out=min(4, Ci // 16), core_bits=16)
    err, row = _full_compare(dqm, L)
    _say(f"bf16 cores {case}: rel err {err:.2e} worst row {row:.2e}")


# The core GEMM's last, partly filled round split along K: layers of a few
# tiles with long K loops run every tile as K-chunk units whose partials a
# second kernel sums.  Chunks of unequal length (17 FP8 steps in 5 chunks:
# 3, 3, 4, 3, 4), FP4 cores (40 steps), bf16 cores (68 steps of 32 channels,
# the walk's 8-tile groups), channels not a multiple of 128.
KSPLIT = [
    # T, H, W, cube, Ci, Co, rank, dtype, core bits
    (3, 16, 16, (1, 2, 2), 2176, 512, 32, "bf16", 8),
    (2, 16, 16, (2, 2, 2), 5120, 320, 32, "bf16", 4),
    (3, 16, 16, (1, 2, 2), 2176, 512, 16, "f32", 16),
    (3, 12, 14, (1, 2, 2), 2080, 256, 16, "bf16", 8),
]


@pytest.mark.parametrize("case", KSPLIT, ids=[f"{c[0]}x{c[1]}x{c[2]}_ci{c[4]}_co{c[5]}_core{c[8]}" for c in KSPLIT])
def test_core_term_k_split(dqm, case):
    T, H, W, cube, Ci, Co, rank, dtype, bits = case
    _say(f"case core K split {case}")
    L = _layer(dqm, T, H, W, cube, Ci, Co, rank, dtype, xseed=T * 100 + Ci + 5, wseed=Co + 15,
               n_out=4, core_bits=bits)
    err, row = _full_compare(dqm, L)
    _say(f"core K split {case}: rel err {err:.2e} worst row {row:.2e}")


# The activation pass's channel split: segments whose blocks fill at most
# half of the CUs run each block as 2-8 parts of its channel chunks, and U is
# the bf16 of the parts' fp32 sums in part order.  Every form of the pass:
# one pass (bf16 four-token cubes and the general fp32 form), two phases
# (one 64-token cube per block, two 24-token cubes), a wave per cube
# (16 tokens), eighths (8 tokens), cubes of more than 64 tokens, one-token
# cubes, two frame segments, no low-rank branch, rank 96 (one quantizer
# group), FP4 cores with 64-channel groups, bf16 cores.
CSPLIT = [
    # T, H, W, cube, Ci, Co, rank, dtype, core bits, core group
    (3, 10, 12, (1, 2, 2), 1024, 256, 32, "bf16", 8, 32),
    (3, 10, 12, (1, 2, 2), 512, 256, 32, "f32", 8, 32),
    (4, 8, 16, (4, 2, 8), 2048, 256, 32, "bf16", 8, 32),
    (2, 6, 8, (2, 3, 4), 1024, 128, 16, "bf16", 8, 32),
    (4, 8, 8, (4, 1, 4), 1024, 256, 32, "bf16", 8, 32),
    (4, 6, 8, (2, 2, 2), 1024, 256, 32, "f32", 8, 32),
    (3, 9, 10, (3, 9, 10), 1024, 128, 16, "bf16", 8, 32),
    (2, 5, 6, (1, 1, 1), 1024, 128, 32, "bf16", 8, 32),
    (5, 6, 8, (2, 2, 2), 1024, 256, 32, "bf16", 8, 32),
    (3, 10, 12, (1, 2, 2), 1024, 256, 0, "bf16", 8, 32),
    (3, 10, 12, (1, 2, 2), 1024, 256, 96, "bf16", 8, 32),
    (4, 8, 16, (4, 2, 8), 2048, 256, 32, "bf16", 4, 64),
    (3, 10, 12, (1, 2, 2), 1024, 256, 32, "bf16", 16, 32),
]


@pytest.mark.parametrize("case", CSPLIT, ids=[f"{c[0]}x{c[1]}x{c[2]}_c{'x'.join(map(str, c[3]))}_ci{c[4]}_r{c[6]}_{c[7]}"
                                              f"_core{c[8]}g{c[9]}" for c in CSPLIT])
def test_activation_channel_split(dqm, case):
    T, H, W, cube, Ci, Co, rank, dtype, bits, grp = case
    _say(f"case activation channel split {case}")
    L = _layer(dqm, T, H, W, cube, Ci, Co, rank, dtype, xseed=T * 100 + Ci + 7, wseed=Co + 17,
               n_out=4, core_bits=bits, core_group=grp)
    err, row = _full_compare(dqm, L)
    _say(f"activation channel split {case}: rel err {err:.2e} worst row {row:.2e}")


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
    # a layer of 3 rounds of tiles: dq_linear takes the one-kernel form (its
    # output was checked in full above); the two kernels on the same
    # activation state give the same output (the core GEMM runs one round,
    # every tile forwards: bit-identical)
    assert dqm.dq_forward_form(L["weights"], L["qa"]) == "one kernel"
    y2 = torch.full((cfg.N, cfg.Co), float("nan"), device=DEV)
    dqm.dq_core_term(L["weights"], L["qa"])
    dqm.dq_delta_term(L["weights"], L["qa"], y2)
    torch.cuda.synchronize()
    a, b = y2.cpu().numpy(), L["y"]
    assert np.isfinite(a).all(), "unwritten outputs (two kernels)"
    d = float(np.linalg.norm(a - b) / np.linalg.norm(b))
    _say(f"wan1p3b_proj: two kernels against the one-kernel form {d:.2e} (bit-identical: {np.array_equal(a, b)})")
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), d


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
    """dq_core_term then dq_delta_term is dq_linear_forward (the same launches;
    with Ci = 256 the one-kernel form does not apply)."""
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


@pytest.mark.parametrize("shape", [(4, 16, 16, 512, 512, "bf16", 32), (3, 10, 18, 1024, 768, "bf16", 32),
                                   (2, 9, 30, 640, 256, "bf16", 32), (3, 7, 22, 576, 512, "f32", 64)],
                         ids=["1024tok_ci512", "540tok_ci1024_ragged", "540tok_ci640_odd_cubes",
                              "462tok_ci576_padded_f32_g64"])
def test_fused_forward_matches_halves(dqm, shape):
    """4-token cubes with FP8 cores: dq_linear_forward_fused runs the one-kernel
    form (core and delta partial sums in one K loop), dq_core_term +
    dq_delta_term the two-kernel form.  Where the core GEMM runs a single
    round (every tile walks K forwards, no K split), both accumulate the same
    MFMA blocks in the same order and add the same terms, so y is
    bit-identical, pad slots and clipped cubes included; the layer also meets
    the oracle's bar."""
    T, H, W, Ci, Co, dtype, core_group = shape
    _say(f"case fused forward {shape}")
    x = synth.make_activation(T, H, W, Ci, seed=25, dtype=dtype, n_outliers=4).to(DEV)
    wt = synth.make_weight(Ci, Co, seed=26, dtype=dtype)
    l1, l2 = _random_factors(Ci, Co, 32, 29)
    weights = dqm.dq_prepare_weights_lowrank(wt, l1, l2)
    qa = dqm.dq_qact_create(weights, (T, H, W, 1, 2, 2), core_group=core_group)
    dqm.dq_quantize_act(weights, x, qa)
    y1 = torch.full((T * H * W, Co), float("nan"), device=DEV)
    y2 = torch.full((T * H * W, Co), float("nan"), device=DEV)
    dqm.dq_linear_forward_fused(weights, qa, y1)
    dqm.dq_core_term(weights, qa)
    dqm.dq_delta_term(weights, qa, y2)
    torch.cuda.synchronize()
    a, b = y1.cpu().numpy(), y2.cpu().numpy()
    assert np.isfinite(a).all()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"max diff {np.abs(a - b).max()}"
    L = dict(x=synth.to_f32_numpy(x.cpu()), wt=synth.to_f32_numpy(wt), l1=l1, l2=l2, weights=weights, qa=qa, y=a,
             g=cubes.Geometry(T, H, W, 1, 2, 2), core_group=core_group)
    err, row = _full_compare(dqm, L)
    _say(f"fused {shape}: rel err {err:.2e} worst row {row:.2e}")


def test_forward_form_choice(dqm):
    """dq_linear_forward takes the one-kernel form for 4-token FP8-core layers
    of at most 16 rounds of 256 x 256 tiles per compute unit, the two kernels
    beyond and wherever the one-kernel form does not apply."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wt = synth.make_weight(512, 8192, seed=46, dtype="bf16")
    l1, l2 = _random_factors(512, 8192, 32, 49)
    weights = dqm.dq_prepare_weights_lowrank(wt, l1, l2)
    for (T, H, W), cube in (((4, 16, 16), (1, 2, 2)), ((4, 96, 96), (1, 2, 2)), ((4, 16, 16), (2, 2, 2))):
        qa = dqm.dq_qact_create(weights, (T, H, W) + cube)
        slots = -(-(T // cube[0]) * -(-H // cube[1]) * -(-W // cube[2]) * cube[0] * cube[1] * cube[2] // 256)
        tiles = (8192 // 256) * slots
        want = "one kernel" if (cube == (1, 2, 2) and tiles <= 16 * cus) else "two kernels"
        _say(f"form {T}x{H}x{W} cube {cube}: {tiles} tiles -> {dqm.dq_forward_form(weights, qa)}")
        assert dqm.dq_forward_form(weights, qa) == want


def test_fused_forward_rejects_other_shapes(dqm):
    """The one-kernel form takes 4-token cubes with FP8 cores only: other
    workspaces are refused with an error, nothing is launched."""
    T, H, W, Ci, Co = 2, 8, 8, 512, 256
    wt = synth.make_weight(Ci, Co, seed=36, dtype="bf16")
    l1, l2 = _random_factors(Ci, Co, 32, 39)
    weights = dqm.dq_prepare_weights_lowrank(wt, l1, l2)
    y = torch.empty(T * H * W, Co, device=DEV)
    for cube, bits in (((2, 2, 2), 8), ((1, 2, 2), 4), ((1, 2, 2), 16), ((1, 1, 1), 8)):
        qa = dqm.dq_qact_create(weights, (T, H, W) + cube, core_bits=bits)
        with pytest.raises(dqm.DQError):
            dqm.dq_linear_forward_fused(weights, qa, y)

def test_library_svd_path(dqm):
    """dq_prepare_weights: the host SVD factors meet Eckart-Young, and R and
    Q4(R) are those the oracle forms from the library's own factors, bit for
    bit (R = fl32(W - L1 L2) with the product summed in fp64 in rank order,
    then MX-FP4 along Ci)."""
    _say("case library svd")
    Ci, Co, r = 256, 384, 32
    wt = synth.make_weight(Ci, Co, seed=31, dtype="bf16", outlier_rows=3)
    weights = dqm.dq_prepare_weights(wt, r, seed=3)
    e = dqm.dq_weights_export(weights)
    wf = synth.to_f32_numpy(wt)
    s = np.linalg.svd(wf.astype(np.float64), compute_uv=False)
    ey = lowrank.eckart_young_ratio(wf, e["l1"], e["l2"], s)
    assert ey["err"] <= (1 + 1e-3) * ey["best"] + ey["bf16_slack"], ey
    ro = lowrank.residual(wf, e["l1"], e["l2"])
    assert np.array_equal(e["r"].view(np.uint32), ro.view(np.uint32)), "R"
    rc, rs = lowrank.quantize_residual(ro)
    assert np.array_equal(e["rcodes"], rc), "Q4(R) codes"
    assert np.array_equal(e["rscales"], rs), "Q4(R) scale codes"


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


def _workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _compare_every_cube(got, xf, g, chunk=2048):
    """Core codes and scale codes of every cube and delta codes and scale
    codes of every token, against the oracle's steps (cube cores, deltas
    against them, MX encoding: what layer.quantize_activation does), taken in
    chunks of cubes and tokens on a thread pool (numpy releases the GIL in
    the bulk of this work).  Bit-exact."""
    from concurrent.futures import ThreadPoolExecutor

    core = cubes.cube_core(xf, g)

    def cores(k0):
        c, sc = mx.mx_quantize(core[k0:k0 + chunk], "fp8")
        ok = np.array_equal(got["core_codes"][k0:k0 + chunk], c) and np.array_equal(got["core_scales"][k0:k0 + chunk], sc)
        return None if ok else f"core codes or scales differ in cubes [{k0}, {k0 + chunk})"

    def deltas(n0):
        toks = np.arange(n0, min(g.N, n0 + chunk))
        c, sc = mx.mx_quantize(cubes.cube_delta(xf, core, g, toks), "fp4")
        ok = np.array_equal(got["delta_codes"][toks], mx.pack_fp4(c)) and np.array_equal(got["delta_scales"][toks], sc)
        return None if ok else f"delta codes or scales differ in tokens [{n0}, {n0 + chunk})"

    with ThreadPoolExecutor(_workers()) as ex:
        bad = [m for m in ex.map(cores, range(0, g.K, chunk)) if m]
        bad += [m for m in ex.map(deltas, range(0, g.N, chunk)) if m]
    assert not bad, bad[:4]


def _full_size_case(dqm, cfg, cube, xseed, check_weights, n_cubes=48, max_rows=512, versus_direct=False,
                    every_cube=True, other_form=False):
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
    xf = synth.to_f32_numpy(x)
    if every_cube:
        _say(f"case {cfg.name} cube {cube}: codes of every cube against the oracle")
        _compare_every_cube(got, xf, g)
    ids = _sample_cubes(g, n_cubes, xseed)
    tbl, cnt = cubes.cube_tokens(g, ids)
    toks = np.sort(tbl[tbl >= 0])
    rng = np.random.default_rng(xseed)
    if len(toks) > max_rows:          # keep every partial cube's tokens, sample the rest
        part = np.isin(cubes.cube_of_token(g, toks), ids[cnt < g.S])
        keep = np.concatenate([toks[part][:max_rows // 2],
                               rng.choice(toks[~part], size=max_rows - min(part.sum(), max_rows // 2), replace=False)])
        toks = np.sort(keep)
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
    if other_form:
        # the form of the forward dq_linear did not take (one kernel, or the
        # two kernels), on the same activation state: the oracle's bar on the
        # sampled tokens, and against dq_linear's output on every element (the
        # core GEMM's odd tiles sum K backwards, so the two may differ in the
        # order of the core term's fp32 additions)
        form = dqm.dq_forward_form(weights, qa)
        y2 = torch.full((cfg.N, cfg.Co), float("nan"), device=DEV)
        if form == "one kernel":
            dqm.dq_core_term(weights, qa)
            dqm.dq_delta_term(weights, qa, y2)
        else:
            dqm.dq_linear_forward_fused(weights, qa, y2)
        torch.cuda.synchronize()
        assert not torch.isnan(y2).any().item(), "unwritten outputs (other form)"
        err2, row2 = _check_y(y2.cpu().numpy()[q["tokens"]], yo, bound)
        d = (torch.linalg.vector_norm(y2 - y) / torch.linalg.vector_norm(y)).item()
        same = torch.equal(y2, y)
        _say(f"{cfg.name} cube {cube}: dq_linear took {form}; the other form Y rel err {err2:.2e} worst row "
             f"{row2:.2e}, against dq_linear {d:.2e} over all outputs (bit-identical: {same})")
        assert d <= 1e-6, d
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


def test_attn14b_projection_4token_cubes(dqm):
    """The 14B attention projection with 4-token cubes: 9.5 rounds of tiles,
    so dq_linear takes the one-kernel forward; checked against the oracle on
    sampled cubes and against the two kernels on every output."""
    cfg = synth.CONFIGS["attn14b_proj"]
    _full_size_case(dqm, cfg, (1, 2, 2), cfg.x_seeds[0], check_weights=False, n_cubes=24, other_form=True)


def test_ffn_up_720p_sampled(dqm):
    cfg = synth.CONFIGS["ffn_up_720p"]
    _full_size_case(dqm, cfg, cfg.cubes[0], cfg.x_seeds[0], check_weights=True, other_form=True)


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
