"""GPU parity of the rotated-basis W4A4 layers (OrbitQuant notes: RPBH
rotation, Lloyd-Max codebook; weights rotated and coded offline, activations
online) through the C ABI against oracle/orbit.py.

Bit-exact: the bf16 codebooks (the library derives its own Lloyd-Max levels
in C++), the weight's and the activations' level indices and row scales (the
rotation's fp32 butterflies and the RMS order are fixed, so the GPU and the
oracle take every coding decision on the same fp32 values).  y: relative
Frobenius error <= 2e-3, every element inside the bound of the bf16 MFMA
contraction (the decoded levels are exact bf16 values; fp32 accumulation of
16-term blocks), every row within ROW_TOL.
"""
import numpy as np
import pytest
import torch

from oracle import layer, lowrank, mx, orbit
from parity_util import DEV, ROW_TOL, TOL, _say
from w4a4_quantized_linear_cube_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dqm(lib):
    from w4a4_quantized_linear_cube_amd import dq
    return dq


def _run(dqm, x, wt, perm, wbits, abits):
    o = dqm.dq_orbit_prepare(wt, perm, wbits, abits)
    N = x.shape[0]
    a = dqm.dq_orbit_act_create(o, N)
    y = torch.full((N, wt.shape[0]), float("nan"), device=DEV)
    dqm.dq_orbit_linear(o, x.to(DEV), a, y)
    torch.cuda.synchronize()
    return o, a, y.cpu().numpy()


def _compare(dqm, o, a, y, xf, wf, perm, wbits, abits, rows=None, chunk=2048):
    cbw, cba = orbit.codebook_bf16(wbits), orbit.codebook_bf16(abits)
    e = dqm.dq_orbit_export(o)
    assert np.array_equal(e["wlev"], cbw), ("weight codebook", e["wlev"], cbw)
    assert np.array_equal(e["alev"], cba), ("activation codebook", e["alev"], cba)
    qw = orbit.quantize_rows(wf, perm, cbw)
    assert np.array_equal(e["wscale"].view(np.uint32), qw["scale"].view(np.uint32)), "weight row scales"
    assert np.array_equal(e["wcodes"], qw["packed"]), "weight codes"
    got = dqm.dq_orbit_act_export(a)
    for n0 in range(0, xf.shape[0], chunk):                    # activations in chunks (memory)
        q = orbit.quantize_rows(xf[n0:n0 + chunk], perm, cba)
        assert np.array_equal(got["scale"][n0:n0 + chunk].view(np.uint32), q["scale"].view(np.uint32)), "token scales"
        assert np.array_equal(got["codes"][n0:n0 + chunk], q["packed"]), f"token codes in [{n0}, {n0 + chunk})"
    sel = np.arange(xf.shape[0]) if rows is None else np.asarray(rows)
    qx = orbit.quantize_rows(xf[sel], perm, cba)
    yo = orbit.forward(qx, qw, cba, cbw).astype(np.float64)
    ys = y[sel].astype(np.float64)
    assert not np.isnan(ys).any(), "unwritten outputs"
    err = layer.rel_fro(ys, yo)
    assert err <= TOL, err
    num, den = np.linalg.norm(ys - yo, axis=1), np.linalg.norm(yo, axis=1)
    live = den > 0
    row = float((num[live] / den[live]).max()) if live.any() else 0.0
    assert row <= ROW_TOL, row
    lx = np.abs(mx.bf16_bits_to_f64(cba)[qx["codes"]])
    lw = np.abs(mx.bf16_bits_to_f64(cbw)[qw["codes"]])
    blocks = xf.shape[1] // 16 + 4
    lim = (blocks * 2.0 ** -23) * (lx @ lw.T) * qx["scale"][:, None] * qw["scale"][None, :] + 3 * 2.0 ** -24 * np.abs(yo) \
        + 1e-30
    bad = np.argwhere(np.abs(ys - yo) > lim)
    assert len(bad) == 0, f"{len(bad)} outputs outside the bound, first {bad[:5]}"
    return err, row


CASES = [
    # N, Ci, Co, wbits, abits, dtype
    (300, 256, 512, 4, 4, "bf16"),
    (77, 512, 200, 4, 4, "f32"),       # Co off the tile size
    (513, 768, 256, 2, 4, "bf16"),     # W2A4, a second row tile
    (64, 1024, 96, 3, 3, "f32"),
    (1, 256, 48, 4, 2, "f32"),
    (40, 15360, 64, 4, 4, "f32"),      # the largest Ci: the rotation pass holds 120 KB of LDS
    (33, 15360, 40, 3, 4, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"n{c[0]}_ci{c[1]}_co{c[2]}_w{c[3]}a{c[4]}_{c[5]}" for c in CASES])
def test_orbit_small(dqm, case):
    N, Ci, Co, wb, ab, dtype = case
    _say(f"case orbit {case}")
    rng = np.random.default_rng(N + Ci)
    x = synth.make_activation(1, 1, N, Ci, seed=N + 1, dtype=dtype, n_outliers=4)
    xf = synth.to_f32_numpy(x).copy()
    if N > 2:
        xf[1] = 0.0                                        # a zero token (scale 0)
        xf[2] = 0.75                                       # a constant token
        x = torch.from_numpy(xf).to(x.dtype)
    wt = synth.make_weight(Ci, Co, seed=Co + 5, dtype=dtype, outlier_rows=2)
    wf = synth.to_f32_numpy(wt)
    perm = rng.permutation(Ci).astype(np.int32)
    o, a, y = _run(dqm, x, wt, perm, wb, ab)
    err, row = _compare(dqm, o, a, y, xf, wf, perm, wb, ab)
    _say(f"orbit {case}: codes and scales bit-exact; rel err {err:.2e} worst row {row:.2e}")


def test_orbit_rejects_bad_permutations(dqm):
    wt = synth.make_weight(256, 64, seed=1, dtype="f32")
    with pytest.raises(dqm.DQError, match="DQ_ERR_INVALID_ARG"):
        dqm.dq_orbit_prepare(wt, np.zeros(256, np.int32))
    with pytest.raises(dqm.DQError, match="DQ_ERR_INVALID_ARG"):
        dqm.dq_orbit_prepare(wt, np.arange(1, 257, dtype=np.int32))
    with pytest.raises(dqm.DQError, match="DQ_ERR_SHAPE"):
        dqm.dq_orbit_prepare(synth.make_weight(320, 64, seed=1, dtype="f32"), np.arange(320, dtype=np.int32))


def test_orbit_attn14b_shape(dqm):
    """The 14B attention projection's shape (31 200 tokens, 5120 -> 5120):
    codes and scales of every token bit-exact, y on sampled tokens; and the
    output error against the exact X W next to direct MX W4A4 of the same
    weight (no low-rank branch in either)."""
    cfg = synth.CONFIGS["attn14b_proj"]
    _say("case orbit attn14b")
    x = synth.make_activation(cfg.T, cfg.H, cfg.W, cfg.Ci, seed=cfg.x_seeds[0], dtype=cfg.dtype,
                              n_outliers=cfg.n_outliers)
    wt = synth.config_weight(cfg)
    xf, wf = synth.to_f32_numpy(x), synth.to_f32_numpy(wt)
    perm = np.random.default_rng(77).permutation(cfg.Ci).astype(np.int32)
    o, a, y = _run(dqm, x, wt, perm, 4, 4)
    rows = np.sort(np.random.default_rng(3).choice(cfg.N, 256, replace=False))
    err, row = _compare(dqm, o, a, y, xf, wf, perm, 4, 4, rows=rows)
    ex = layer.exact_output(xf[rows], wf)
    e_orbit = layer.rel_fro(y[rows], ex)
    zero_u = np.zeros((len(rows), 0), np.uint16)
    e_mx = layer.rel_fro(layer.direct_output(xf[rows], zero_u, np.zeros((0, cfg.Co), np.uint16),
                                             *lowrank.quantize_residual(wf)), ex)
    _say(f"orbit attn14b: codes bit-exact on {cfg.N} tokens; y rel err {err:.2e} on {len(rows)} rows; "
         f"error vs exact X W: rotated Lloyd-Max W4A4 {e_orbit:.3e}, direct MX W4A4 {e_mx:.3e}")
