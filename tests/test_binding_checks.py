"""The binding's argument checks (no GPU needed).

The C ABI receives raw device pointers and cannot see sizes, so the Python
binding checks every caller-owned tensor before its pointer crosses: shape
against the workspace (x [N][Ci], y [N][Co]), dtype, contiguity, device and
alignment; and the bf16 factors' shapes against (Ci, rank) and (rank, Co).
Each rejection raises DQError before the library is touched, which these
tests show with stand-in handles and CPU tensors.
"""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

from w4a4_quantized_linear_cube_amd import dq

W = SimpleNamespace(Ci=64, Co=96, rank=16, device=0, handle=None)
Q = SimpleNamespace(N=40, weights=W, handle=None)


def _raises(fn, *args, match):
    with pytest.raises(dq.DQError, match=match):
        fn(*args)


@pytest.mark.parametrize("fn", [dq.dq_quantize_act, lambda w, x, q: dq.dq_linear(w, x, q, None)])
def test_x_rejections(fn):
    _raises(fn, W, torch.zeros(40, 64, dtype=torch.float16), Q, match="dtype")
    _raises(fn, W, torch.zeros(41, 64), Q, match="shape")
    _raises(fn, W, torch.zeros(40, 32), Q, match="shape")
    _raises(fn, W, torch.zeros(64, 40).t(), Q, match="contiguous")
    _raises(fn, W, np.zeros((40, 64), np.float32), Q, match="torch tensor")
    _raises(fn, W, torch.zeros(40, 64, dtype=torch.bfloat16), Q, match="cuda:0")     # CPU tensor


@pytest.mark.parametrize("fn", [dq.dq_linear_forward, dq.dq_delta_term, dq.dq_linear_forward_fused])
def test_y_rejections(fn):
    _raises(fn, W, Q, torch.zeros(40, 96, dtype=torch.bfloat16), match="dtype")
    _raises(fn, W, Q, torch.zeros(40, 95), match="shape")
    _raises(fn, W, Q, torch.zeros(39, 96), match="shape")
    _raises(fn, W, Q, torch.zeros(96, 40).t(), match="contiguous")
    _raises(fn, W, Q, torch.zeros(40, 96), match="cuda:0")


def test_dq_linear_checks_y_after_x():
    _raises(dq.dq_linear, W, torch.zeros(40, 64), Q, torch.zeros(40, 96, dtype=torch.float64), match="x is on")


def test_workspace_of_another_weight():
    other = SimpleNamespace(Ci=64, Co=128, rank=16, device=0, handle=None)
    _raises(dq.dq_core_term, other, Q, match="different weight")


def test_factor_rejections():
    w = torch.zeros(96, 64)
    l1 = np.zeros((64, 16), np.uint16)
    l2 = np.zeros((16, 96), np.uint16)
    f = dq.dq_prepare_weights_lowrank
    _raises(f, w, l1, None, match="both factors")
    _raises(f, w, np.zeros((63, 16), np.uint16), l2, match="l1 has shape")
    _raises(f, w, l1, np.zeros((16, 95), np.uint16), match="l2 has shape")
    _raises(f, w, l1, np.zeros((8, 96), np.uint16), match="l2 has shape")
    _raises(f, w, l1.astype(np.float32), l2, match="bf16 bits")
    _raises(f, w, np.zeros(64, np.uint16), l2, match="2-D")
    _raises(f, torch.zeros(96), l1, l2, match="2-D")
