"""Python binding of libdq.so (include/dq.h): argument marshalling only.

Every function here has the name of the C entry point it calls.  Device
tensors are torch tensors on the handle's device (PyTorch supplies memory and
streams); host arrays are numpy.  No arithmetic of the layer happens here, and
there is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

DQ_F32, DQ_BF16 = 0, 1
STATUS = {0: "DQ_OK", 1: "DQ_ERR_INVALID_ARG", 2: "DQ_ERR_SHAPE", 3: "DQ_ERR_UNSUPPORTED",
          4: "DQ_ERR_OUT_OF_MEMORY", 5: "DQ_ERR_DEVICE"}

# every entry point declared in include/dq.h
EXPORTS = ("dq_last_error", "dq_status_str", "dq_lowrank_factors", "dq_prepare_weights_lowrank",
           "dq_prepare_weights", "dq_weights_destroy", "dq_weights_info", "dq_weights_export",
           "dq_qact_create", "dq_qact_create_ex", "dq_qact_destroy", "dq_qact_info", "dq_quantize_act", "dq_linear_forward",
           "dq_core_term", "dq_delta_term", "dq_linear", "dq_qact_export")


class DQError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        super().__init__(f"{func}: {STATUS.get(status, status)}: {msg}")
        self.status = status


class Geom(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "H", "W", "t", "h", "w")]


def library_path() -> str:
    return os.path.join(_HERE, "libdq.so")


def load():
    """Load libdq.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P, I32, I64, U64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
    PP = ctypes.POINTER(ctypes.c_void_p)
    sig = {
        "dq_last_error": ([], ctypes.c_char_p),
        "dq_status_str": ([ctypes.c_int], ctypes.c_char_p),
        "dq_lowrank_factors": ([P, ctypes.c_int, I64, I64, I32, U64, P, P], ctypes.c_int),
        "dq_prepare_weights_lowrank": ([P, ctypes.c_int, I64, I64, I32, P, P, I32, PP], ctypes.c_int),
        "dq_prepare_weights": ([P, ctypes.c_int, I64, I64, I32, U64, I32, PP], ctypes.c_int),
        "dq_weights_destroy": ([P], None),
        "dq_weights_info": ([P, P, P, P, P], ctypes.c_int),
        "dq_weights_export": ([P, P, P, P, P, P], ctypes.c_int),
        "dq_qact_create": ([P, Geom, PP], ctypes.c_int),
        "dq_qact_create_ex": ([P, Geom, I32, I32, PP], ctypes.c_int),
        "dq_qact_destroy": ([P], None),
        "dq_qact_info": ([P, P, P, P], ctypes.c_int),
        "dq_quantize_act": ([P, P, ctypes.c_int, P, P], ctypes.c_int),
        "dq_linear_forward": ([P, P, P, P], ctypes.c_int),
        "dq_core_term": ([P, P, P], ctypes.c_int),
        "dq_delta_term": ([P, P, P, P], ctypes.c_int),
        "dq_linear": ([P, P, ctypes.c_int, P, P, P], ctypes.c_int),
        "dq_qact_export": ([P, P, P, P, P, P, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _LIB = lib
    return lib


def _check(status: int, func: str):
    if status != 0:
        raise DQError(status, func, load().dq_last_error().decode())


def _ptr(a) -> ctypes.c_void_p:
    if a is None:
        return ctypes.c_void_p(None)
    if isinstance(a, np.ndarray):
        return ctypes.c_void_p(a.ctypes.data)
    return ctypes.c_void_p(a.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(getattr(stream, "cuda_stream", stream))


def _dtype_of(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return DQ_BF16
    if t.dtype == torch.float32:
        return DQ_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _host_weight(w):
    """W^T [Co][Ci] as a contiguous CPU torch tensor; returns (tensor, dtype code)."""
    import torch
    w = w.detach().to("cpu").contiguous()
    return w, _dtype_of(w)


class Weights:
    """Owns a dq_weights handle."""

    def __init__(self, handle: ctypes.c_void_p):
        self.handle = handle
        Ci, Co, r, dev = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
        _check(load().dq_weights_info(handle, ctypes.byref(Ci), ctypes.byref(Co), ctypes.byref(r), ctypes.byref(dev)),
               "dq_weights_info")
        self.Ci, self.Co, self.rank, self.device = Ci.value, Co.value, r.value, dev.value

    def __del__(self):
        if getattr(self, "handle", None) and _LIB is not None:
            _LIB.dq_weights_destroy(self.handle)
            self.handle = None


class QAct:
    """Owns a dq_qact handle (keeps its weights alive)."""

    def __init__(self, handle: ctypes.c_void_p, weights: Weights, geom: Tuple[int, ...], core_bits: int = 8):
        self.handle = handle
        self.weights = weights
        self.geom = tuple(geom)
        self.core_bits = core_bits
        N, K, nb = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(load().dq_qact_info(handle, ctypes.byref(N), ctypes.byref(K), ctypes.byref(nb)), "dq_qact_info")
        self.N, self.K, self.device_bytes = N.value, K.value, nb.value

    def __del__(self):
        if getattr(self, "handle", None) and _LIB is not None:
            _LIB.dq_qact_destroy(self.handle)
            self.handle = None


def dq_lowrank_factors(w, rank: int, seed: int):
    """Host SVD factors: returns (L1 bits uint16 [Ci][rank], L2 bits uint16 [rank][Co])."""
    wt, dt = _host_weight(w)
    Co, Ci = wt.shape
    l1 = np.zeros((Ci, rank), dtype=np.uint16)
    l2 = np.zeros((rank, Co), dtype=np.uint16)
    _check(load().dq_lowrank_factors(_ptr(wt), dt, Ci, Co, rank, seed, _ptr(l1), _ptr(l2)), "dq_lowrank_factors")
    return l1, l2


def dq_prepare_weights_lowrank(w, l1: Optional[np.ndarray], l2: Optional[np.ndarray], device: int = 0) -> Weights:
    wt, dt = _host_weight(w)
    Co, Ci = wt.shape
    rank = 0 if l1 is None else l1.shape[1]
    l1c = None if l1 is None else np.ascontiguousarray(l1, dtype=np.uint16)
    l2c = None if l2 is None else np.ascontiguousarray(l2, dtype=np.uint16)
    h = ctypes.c_void_p()
    _check(load().dq_prepare_weights_lowrank(_ptr(wt), dt, Ci, Co, rank, _ptr(l1c), _ptr(l2c), device,
                                             ctypes.byref(h)), "dq_prepare_weights_lowrank")
    return Weights(h)


def dq_prepare_weights(w, rank: int, seed: int = 0, device: int = 0) -> Weights:
    wt, dt = _host_weight(w)
    Co, Ci = wt.shape
    h = ctypes.c_void_p()
    _check(load().dq_prepare_weights(_ptr(wt), dt, Ci, Co, rank, seed, device, ctypes.byref(h)), "dq_prepare_weights")
    return Weights(h)


def dq_weights_export(w: Weights) -> dict:
    Ci, Co, r = w.Ci, w.Co, w.rank
    out = dict(l1=np.zeros((Ci, r), np.uint16), l2=np.zeros((r, Co), np.uint16), r=np.zeros((Co, Ci), np.float32),
               rcodes=np.zeros((Co, Ci // 2), np.uint8), rscales=np.zeros((Co, Ci // 32), np.uint8))
    _check(load().dq_weights_export(w.handle, _ptr(out["l1"]), _ptr(out["l2"]), _ptr(out["r"]), _ptr(out["rcodes"]),
                                    _ptr(out["rscales"])), "dq_weights_export")
    return out


def dq_qact_create(w: Weights, geom: Sequence[int], core_group: int = 32, core_bits: int = 8) -> QAct:
    """Workspace for a (T, H, W, t, h, w) geometry; core_group 64 gives the
    cores one scale per 64 channels, core_bits 4 MX-FP4 cores
    (dq_qact_create_ex)."""
    h = ctypes.c_void_p()
    if core_group == 32 and core_bits == 8:
        _check(load().dq_qact_create(w.handle, Geom(*geom), ctypes.byref(h)), "dq_qact_create")
    else:
        _check(load().dq_qact_create_ex(w.handle, Geom(*geom), core_group, core_bits, ctypes.byref(h)),
               "dq_qact_create_ex")
    return QAct(h, w, geom, core_bits)


def dq_quantize_act(w: Weights, x, q: QAct, stream=None):
    _check(load().dq_quantize_act(w.handle, _ptr(x), _dtype_of(x), q.handle, _stream(stream)), "dq_quantize_act")


def dq_linear_forward(w: Weights, q: QAct, y, stream=None):
    _check(load().dq_linear_forward(w.handle, q.handle, _ptr(y), _stream(stream)), "dq_linear_forward")


def dq_core_term(w: Weights, q: QAct, stream=None):
    _check(load().dq_core_term(w.handle, q.handle, _stream(stream)), "dq_core_term")


def dq_delta_term(w: Weights, q: QAct, y, stream=None):
    _check(load().dq_delta_term(w.handle, q.handle, _ptr(y), _stream(stream)), "dq_delta_term")


def dq_linear(w: Weights, x, q: QAct, y, stream=None):
    _check(load().dq_linear(w.handle, _ptr(x), _dtype_of(x), q.handle, _ptr(y), _stream(stream)), "dq_linear")


def dq_qact_export(q: QAct, stream=None) -> dict:
    w = q.weights
    N, K, Ci, r = q.N, q.K, w.Ci, w.rank
    bf16 = q.core_bits == 16                      # bf16 cores: their bits, no scales
    out = dict(delta_codes=np.zeros((N, Ci // 2), np.uint8), delta_scales=np.zeros((N, Ci // 32), np.uint8),
               core_codes=np.zeros((K, Ci), np.uint16 if bf16 else np.uint8),
               core_scales=None if bf16 else np.zeros((K, Ci // 32), np.uint8),
               U=np.zeros((N, r), np.uint16))
    _check(load().dq_qact_export(q.handle, _ptr(out["delta_codes"]), _ptr(out["delta_scales"]),
                                 _ptr(out["core_codes"]), _ptr(out["core_scales"]) if not bf16 else None, _ptr(out["U"]),
                                 _stream(stream)),
           "dq_qact_export")
    return out
