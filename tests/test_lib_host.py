"""Host-side checks of the C-ABI library that need no GPU: it loads, exports
every entry point include/dq.h declares, rejects bad arguments before
touching a device, and its host SVD (the weight split of 关键设计 4) meets
the Eckart-Young bound against LAPACK."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from conftest import gpu_available
from oracle import lowrank
from w4a4_quantized_linear_cube_amd import dq

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dq.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(dq_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert sorted(dq.EXPORTS) == _declared()


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    for code in range(6):
        assert lib.dq_status_str(code).decode()


def _expect(status, code, lib):
    assert status == code, (status, lib.dq_last_error().decode())
    assert lib.dq_last_error().decode()


def test_argument_errors_before_any_device_work(lib):
    w = np.zeros((64, 96), dtype=np.float32)
    l1 = np.zeros((96, 8), np.uint16)
    l2 = np.zeros((8, 64), np.uint16)
    h = ctypes.c_void_p()
    P = lambda a: ctypes.c_void_p(a.ctypes.data)
    # Ci not a multiple of 32
    _expect(lib.dq_prepare_weights_lowrank(P(w), 0, 48, 64, 8, P(l1), P(l2), 0, ctypes.byref(h)), 2, lib)
    # null weight
    _expect(lib.dq_prepare_weights_lowrank(None, 0, 96, 64, 8, P(l1), P(l2), 0, ctypes.byref(h)), 1, lib)
    # rank above min(Ci, Co)
    _expect(lib.dq_prepare_weights_lowrank(P(w), 0, 96, 64, 65, P(l1), P(l2), 0, ctypes.byref(h)), 1, lib)
    # unknown dtype
    _expect(lib.dq_prepare_weights_lowrank(P(w), 7, 96, 64, 8, P(l1), P(l2), 0, ctypes.byref(h)), 1, lib)
    # null factor with rank > 0
    _expect(lib.dq_prepare_weights_lowrank(P(w), 0, 96, 64, 8, None, P(l2), 0, ctypes.byref(h)), 1, lib)
    # workspace for a null weight, and null handles for the hot calls
    _expect(lib.dq_qact_create(None, dq.Geom(2, 2, 2, 1, 1, 1), ctypes.byref(h)), 1, lib)
    _expect(lib.dq_qact_create_ex(None, dq.Geom(2, 2, 2, 1, 1, 1), 64, 8, ctypes.byref(h)), 1, lib)
    _expect(lib.dq_quantize_act(None, None, 0, None, None), 1, lib)
    _expect(lib.dq_linear_forward(None, None, None, None), 1, lib)
    _expect(lib.dq_core_term(None, None, None), 1, lib)
    _expect(lib.dq_delta_term(None, None, None, None), 1, lib)
    _expect(lib.dq_linear_forward_fused(None, None, None, None), 1, lib)
    _expect(lib.dq_forward_form(None, None, None), 1, lib)
    _expect(lib.dq_lowrank_factors(P(w), 0, 96, 64, -1, 0, P(l1), P(l2)), 1, lib)
    _expect(lib.dq_lowrank_factors(P(w), 0, 0, 64, 1, 0, P(l1), P(l2)), 2, lib)


@pytest.mark.skipif(gpu_available(), reason="checks the no-device error path")
def test_no_device_is_reported(lib):
    w = np.zeros((64, 96), dtype=np.float32)
    h = ctypes.c_void_p()
    st = lib.dq_prepare_weights_lowrank(ctypes.c_void_p(w.ctypes.data), 0, 96, 64, 0, None, None, 0, ctypes.byref(h))
    assert st in (1, 5), lib.dq_last_error().decode()     # no HIP device: never a crash


def _planted(Ci, Co, decay, seed):
    rng = np.random.default_rng(seed)
    u, _ = np.linalg.qr(rng.standard_normal((Ci, min(Ci, Co))))
    v, _ = np.linalg.qr(rng.standard_normal((Co, min(Ci, Co))))
    sig = 4.0 * decay ** np.arange(min(Ci, Co))
    return ((u * sig) @ v.T).T.astype(np.float32)      # W^T [Co][Ci]


@pytest.mark.parametrize("shape,rank,dtype", [((256, 192), 16, "f32"), ((128, 320), 32, "bf16"), ((96, 64), 8, "f32")])
def test_host_svd_eckart_young(lib, shape, rank, dtype):
    Ci, Co = shape
    wt = torch.from_numpy(_planted(Ci, Co, 0.85, seed=Ci + Co))
    if dtype == "bf16":
        wt = wt.to(torch.bfloat16)
    wf = wt.float().numpy()
    l1, l2 = dq.dq_lowrank_factors(wt, rank, seed=5)
    s = np.linalg.svd(wf.astype(np.float64), compute_uv=False)
    ey = lowrank.eckart_young_ratio(wf, l1, l2, s)
    assert ey["err"] <= (1 + 1e-3) * ey["best"] + ey["bf16_slack"], ey
    assert ey["captured"] >= 0.99 * ey["top_energy"], ey
    l1b, l2b = dq.dq_lowrank_factors(wt, rank, seed=5)
    assert np.array_equal(l1, l1b) and np.array_equal(l2, l2b)      # deterministic


def test_host_svd_takes_outlier_channels(lib):
    from w4a4_quantized_linear_cube_amd import synth
    wt = synth.make_weight(256, 256, seed=1500, dtype="f32", outlier_rows=2, outlier_factor=10.0)
    l1, l2 = dq.dq_lowrank_factors(wt, 16, seed=1)
    wf = wt.numpy()
    s = np.linalg.svd(wf.astype(np.float64), compute_uv=False)
    ey = lowrank.eckart_young_ratio(wf, l1, l2, s)
    assert ey["err"] <= (1 + 1e-3) * ey["best"] + ey["bf16_slack"], ey
    r = lowrank.residual(wf, l1, l2)
    norms = np.linalg.norm(r, axis=1)
    assert norms.max() < 2.0 * np.median(norms)


def test_rank_zero_factors(lib):
    w = torch.zeros(64, 96)
    l1, l2 = dq.dq_lowrank_factors(w, 0, seed=0)
    assert l1.shape == (96, 0) and l2.shape == (0, 64)
