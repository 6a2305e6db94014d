"""dq_linear_noalloc (the entry point for callers that cannot allocate)
against dq_linear, through the C ABI.

Both run the same kernels on the same input, so their outputs must agree bit
for bit.  The calls come in a row on one GPU, each later one on a smaller or
differently shaped layer, so the fixed scratch array holds the previous
call's bytes when the next one starts: a state that is not cleared or
rewritten would show as a difference.  The second layer has Ci = 192 (channel
padding up to 256, which the entry point must clear) and cubes of more than
64 tokens (block partials), the third one-token cubes, the fourth a core GEMM
split along K (K-chunk partials in the array); then the first layer again.
"""
import ctypes

import numpy as np
import pytest
import torch

from parity_util import DEV, _random_factors, _say
from w4a4_quantized_linear_cube_amd import synth

pytestmark = pytest.mark.gpu

LAYERS = [
    # (T, H, W, cube, Ci, Co, rank, dtype)
    (4, 12, 14, (1, 2, 2), 512, 768, 32, "bf16"),
    (3, 9, 10, (3, 9, 10), 192, 320, 16, "f32"),
    (2, 5, 6, (1, 1, 1), 128, 256, 32, "bf16"),
    (3, 16, 16, (1, 2, 2), 2176, 512, 32, "bf16"),
    (4, 12, 14, (1, 2, 2), 512, 768, 32, "bf16"),
]


@pytest.fixture(scope="module")
def dqm(lib):
    from w4a4_quantized_linear_cube_amd import dq
    return dq


def _bits(t):
    return t.cpu().numpy().view(np.uint32)


def test_noalloc_matches_dq_linear(dqm):
    for i, (T, H, W, cube, Ci, Co, rank, dtype) in enumerate(LAYERS):
        _say(f"case no-alloc call {i}: {T}x{H}x{W} cube {cube} Ci {Ci} Co {Co} rank {rank} {dtype}")
        x = synth.make_activation(T, H, W, Ci, seed=900 + i, dtype=dtype, n_outliers=4).to(DEV)
        wt = synth.make_weight(Ci, Co, seed=950 + i, dtype=dtype)
        l1, l2 = _random_factors(Ci, Co, rank, 970 + i)
        weights = dqm.dq_prepare_weights_lowrank(wt, l1, l2)
        geom = (T, H, W) + tuple(cube)
        qa = dqm.dq_qact_create(weights, geom)
        y_ref = torch.full((T * H * W, Co), float("nan"), device=DEV)
        y = torch.full((T * H * W, Co), float("nan"), device=DEV)
        dqm.dq_linear(weights, x, qa, y_ref)
        dqm.dq_linear_noalloc(weights, x, geom, y)
        torch.cuda.synchronize()
        assert not torch.isnan(y).any().item(), "unwritten outputs"
        assert np.array_equal(_bits(y), _bits(y_ref)), f"call {i}: outputs differ from dq_linear"
        _say(f"no-alloc call {i}: bit-identical to dq_linear")


def test_noalloc_rejects_layers_beyond_the_scratch(dqm, lib):
    """A layer that needs more than the fixed array is refused before any
    device work, with the size it needs."""
    wt = synth.make_weight(5120, 1024, seed=5, dtype="bf16")
    weights = dqm.dq_prepare_weights_lowrank(wt, None, None)
    x = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    y = torch.zeros(16, dtype=torch.float32, device=DEV)
    st = lib.dq_linear_noalloc(weights.handle, ctypes.c_void_p(x.data_ptr()), 1, dqm.Geom(21, 45, 80, 1, 2, 2),
                               ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 2, st
    msg = lib.dq_last_error().decode()
    assert "bytes of scratch" in msg, msg


def test_noalloc_graph_replays(dqm):
    """dq_linear_noalloc captured into a HIP graph (the callers it is for) and
    replayed three times, with an eager call on another input and
    synchronizations between the replays: every replay's output, and every
    eager output, is bit for bit the first eager call's on the same input.
    The layer's core GEMM runs split along K (a kernel of partials, then
    their sum)."""
    T, H, W, cube, Ci, Co, rank, dtype = (3, 16, 16, (1, 2, 2), 2176, 512, 32, "bf16")
    _say(f"case no-alloc graph: {T}x{H}x{W} cube {cube} Ci {Ci} Co {Co} rank {rank} {dtype}")
    x = synth.make_activation(T, H, W, Ci, seed=990, dtype=dtype, n_outliers=4).to(DEV)
    x2 = synth.make_activation(T, H, W, Ci, seed=991, dtype=dtype, n_outliers=4).to(DEV)
    wt = synth.make_weight(Ci, Co, seed=992, dtype=dtype)
    l1, l2 = _random_factors(Ci, Co, rank, 993)
    weights = dqm.dq_prepare_weights_lowrank(wt, l1, l2)
    geom = (T, H, W) + tuple(cube)
    N = T * H * W
    nan = float("nan")
    y_ref = torch.full((N, Co), nan, device=DEV)
    y_ref2 = torch.full((N, Co), nan, device=DEV)
    dqm.dq_linear_noalloc(weights, x, geom, y_ref)          # first call on the device: outside the capture
    dqm.dq_linear_noalloc(weights, x2, geom, y_ref2)
    torch.cuda.synchronize()
    assert not torch.isnan(y_ref).any().item() and not torch.isnan(y_ref2).any().item(), "unwritten outputs"
    y = torch.full((N, Co), nan, device=DEV)
    y2 = torch.full((N, Co), nan, device=DEV)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s, capture_error_mode="thread_local"):
        dqm.dq_linear_noalloc(weights, x, geom, y)
    torch.cuda.synchronize()
    for i in range(3):
        y.fill_(nan)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(y), _bits(y_ref)), f"replay {i}: outputs differ from the eager call"
        y2.fill_(nan)
        dqm.dq_linear_noalloc(weights, x2, geom, y2)      # eager work between replays, on the same array
        torch.cuda.synchronize()
        assert np.array_equal(_bits(y2), _bits(y_ref2)), f"eager call after replay {i}: outputs differ"
    _say("no-alloc graph: three replays bit-identical to the eager call")
