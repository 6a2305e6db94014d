"""Python binding of libdq.so (include/dq.h): argument marshalling only.

Every function here has the name of the C entry point it calls.  Device
tensors are torch tensors on the handle's device (PyTorch supplies memory and
streams); host arrays are numpy.  No arithmetic of the layer happens here, and
there is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from types import SimpleNamespace
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
           "dq_core_term", "dq_delta_term", "dq_linear_forward_fused", "dq_forward_form", "dq_linear", "dq_qact_export", "dq_linear_noalloc",
           "dq_prepare_weights_w6", "dq_act6_create", "dq_act6_destroy", "dq_quantize_act6", "dq_linear6_forward",
           "dq_linear6", "dq_act6_export", "dq_orbit_prepare", "dq_orbit_destroy", "dq_orbit_export",
           "dq_orbit_act_create", "dq_orbit_act_destroy", "dq_orbit_quantize_act", "dq_orbit_forward", "dq_orbit_linear",
           "dq_orbit_act_export")
DQ_FP6_E2M3, DQ_FP6_E3M2 = 2, 3
FP6_FORMATS = {"fp6_e2m3": DQ_FP6_E2M3, "fp6_e3m2": DQ_FP6_E3M2}


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
        "dq_linear_forward_fused": ([P, P, P, P], ctypes.c_int),
        "dq_forward_form": ([P, P, P], ctypes.c_int),
        "dq_linear": ([P, P, ctypes.c_int, P, P, P], ctypes.c_int),
        "dq_qact_export": ([P, P, P, P, P, P, P], ctypes.c_int),
        "dq_linear_noalloc": ([P, P, ctypes.c_int, Geom, P, P], ctypes.c_int),
        "dq_prepare_weights_w6": ([P, ctypes.c_int, I64, I64, I32, P, P, I32, I32, PP], ctypes.c_int),
        "dq_act6_create": ([P, I64, PP], ctypes.c_int),
        "dq_act6_destroy": ([P], None),
        "dq_quantize_act6": ([P, P, ctypes.c_int, P, P], ctypes.c_int),
        "dq_linear6_forward": ([P, P, P, P], ctypes.c_int),
        "dq_linear6": ([P, P, ctypes.c_int, P, P, P], ctypes.c_int),
        "dq_act6_export": ([P, P, P, P, P], ctypes.c_int),
        "dq_orbit_prepare": ([P, ctypes.c_int, I64, I64, P, I32, I32, I32, PP], ctypes.c_int),
        "dq_orbit_destroy": ([P], None),
        "dq_orbit_export": ([P, P, P, P, P], ctypes.c_int),
        "dq_orbit_act_create": ([P, I64, PP], ctypes.c_int),
        "dq_orbit_act_destroy": ([P], None),
        "dq_orbit_quantize_act": ([P, P, ctypes.c_int, P, P], ctypes.c_int),
        "dq_orbit_forward": ([P, P, P, P], ctypes.c_int),
        "dq_orbit_linear": ([P, P, ctypes.c_int, P, P, P], ctypes.c_int),
        "dq_orbit_act_export": ([P, P, P, P], ctypes.c_int),
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
    if not isinstance(w, torch.Tensor) or w.dim() != 2:
        raise DQError(1, "weight", "the weight must be a 2-D torch tensor [Co][Ci]")
    w = w.detach().to("cpu").contiguous()
    return w, _dtype_of(w)


def _invalid(func: str, msg: str):
    raise DQError(1, func, msg)


def _device_tensor(func: str, name: str, t, shape, dtypes, device: int, align: int):
    """Checks a caller-owned device buffer before its pointer crosses the C ABI,
    which cannot see sizes: a torch tensor of one of `dtypes`, exactly `shape`,
    contiguous, on CUDA device `device`, its data `align`-byte aligned."""
    import torch
    if not isinstance(t, torch.Tensor):
        _invalid(func, f"{name} must be a torch tensor")
    if t.dtype not in dtypes:
        _invalid(func, f"{name} has dtype {t.dtype}; expected one of {[str(d) for d in dtypes]}")
    if tuple(t.shape) != tuple(shape):
        _invalid(func, f"{name} has shape {tuple(t.shape)}; expected {tuple(shape)}")
    if not t.is_contiguous():
        _invalid(func, f"{name} must be contiguous")
    if t.device.type != "cuda" or t.device.index != device:
        _invalid(func, f"{name} is on {t.device}; expected cuda:{device}")
    if t.data_ptr() % align:
        _invalid(func, f"{name} must be {align}-byte aligned")


def _check_x(func: str, w: "Weights", q: "QAct", x):
    import torch
    _device_tensor(func, "x", x, (q.N, w.Ci), (torch.bfloat16, torch.float32), w.device, 16)


def _check_y(func: str, w: "Weights", q: "QAct", y):
    import torch
    _device_tensor(func, "y", y, (q.N, w.Co), (torch.float32,), w.device, 4)


def _check_pair(func: str, w: "Weights", q: "QAct"):
    if q.weights is not w and (q.weights.Ci, q.weights.Co, q.weights.rank) != (w.Ci, w.Co, w.rank):
        _invalid(func, "the workspace was created for a different weight")


def _factor(func: str, name: str, a, shape):
    """A bf16 factor given as uint16 (or int16) bits of exactly `shape`."""
    a = np.asarray(a)
    if a.dtype not in (np.uint16, np.int16):
        _invalid(func, f"{name} must hold bf16 bits as uint16 (got {a.dtype})")
    if a.shape != tuple(shape):
        _invalid(func, f"{name} has shape {a.shape}; expected {tuple(shape)}")
    return np.ascontiguousarray(a.view(np.uint16))


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


class Act6:
    """Owns a dq_act6 handle (keeps its weights alive)."""

    def __init__(self, handle: ctypes.c_void_p, weights: "Weights", N: int):
        self.handle = handle
        self.weights = weights
        self.N = N

    def __del__(self):
        if getattr(self, "handle", None) and _LIB is not None:
            _LIB.dq_act6_destroy(self.handle)
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
    f = "dq_prepare_weights_lowrank"
    wt, dt = _host_weight(w)
    Co, Ci = wt.shape
    if (l1 is None) != (l2 is None):
        _invalid(f, "give both factors or neither")
    rank = 0 if l1 is None else np.asarray(l1).shape[-1]
    if l1 is not None and np.asarray(l1).ndim != 2:
        _invalid(f, "l1 must be 2-D [Ci][rank]")
    l1c = None if l1 is None else _factor(f, "l1", l1, (Ci, rank))
    l2c = None if l2 is None else _factor(f, "l2", l2, (rank, Co))
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
    cbytes = Ci // 4 * 3 if getattr(w, "fp6_format", None) else Ci // 2
    out = dict(l1=np.zeros((Ci, r), np.uint16), l2=np.zeros((r, Co), np.uint16), r=np.zeros((Co, Ci), np.float32),
               rcodes=np.zeros((Co, cbytes), np.uint8), rscales=np.zeros((Co, Ci // 32), np.uint8))
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
    _check_pair("dq_quantize_act", w, q)
    _check_x("dq_quantize_act", w, q, x)
    _check(load().dq_quantize_act(w.handle, _ptr(x), _dtype_of(x), q.handle, _stream(stream)), "dq_quantize_act")


def dq_linear_forward(w: Weights, q: QAct, y, stream=None):
    _check_pair("dq_linear_forward", w, q)
    _check_y("dq_linear_forward", w, q, y)
    _check(load().dq_linear_forward(w.handle, q.handle, _ptr(y), _stream(stream)), "dq_linear_forward")


def dq_core_term(w: Weights, q: QAct, stream=None):
    _check_pair("dq_core_term", w, q)
    _check(load().dq_core_term(w.handle, q.handle, _stream(stream)), "dq_core_term")


def dq_delta_term(w: Weights, q: QAct, y, stream=None):
    _check_pair("dq_delta_term", w, q)
    _check_y("dq_delta_term", w, q, y)
    _check(load().dq_delta_term(w.handle, q.handle, _ptr(y), _stream(stream)), "dq_delta_term")


def dq_linear_forward_fused(w: Weights, q: QAct, y, stream=None):
    _check_pair("dq_linear_forward_fused", w, q)
    _check_y("dq_linear_forward_fused", w, q, y)
    _check(load().dq_linear_forward_fused(w.handle, q.handle, _ptr(y), _stream(stream)), "dq_linear_forward_fused")


def dq_forward_form(w: Weights, q: QAct) -> str:
    """'one kernel' or 'two kernels': the form dq_linear_forward takes for this pair."""
    _check_pair("dq_forward_form", w, q)
    flag = ctypes.c_int(0)
    _check(load().dq_forward_form(w.handle, q.handle, ctypes.byref(flag)), "dq_forward_form")
    return "one kernel" if flag.value else "two kernels"


def dq_linear(w: Weights, x, q: QAct, y, stream=None):
    _check_pair("dq_linear", w, q)
    _check_x("dq_linear", w, q, x)
    _check_y("dq_linear", w, q, y)
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


def dq_linear_noalloc(w: Weights, x, geom: Sequence[int], y, stream=None):
    """dq_linear without a workspace handle: the activation state lives in
    the library's fixed per-device array (calls on one GPU must not overlap)."""
    f = "dq_linear_noalloc"
    T, H, W = geom[:3]
    ws = SimpleNamespace(N=T * H * W)
    _check_x(f, w, ws, x)
    _check_y(f, w, ws, y)
    _check(load().dq_linear_noalloc(w.handle, _ptr(x), _dtype_of(x), Geom(*geom), _ptr(y), _stream(stream)), f)


# ---------------------------------------------------------------- 6-bit layers ----
def dq_prepare_weights_w6(w, l1: Optional[np.ndarray], l2: Optional[np.ndarray], fmt: str = "fp6_e2m3",
                          device: int = 0) -> Weights:
    """A 6-bit weight (Q6(R) in MX-FP6 `fmt`: "fp6_e2m3" or "fp6_e3m2")."""
    f = "dq_prepare_weights_w6"
    if fmt not in FP6_FORMATS:
        _invalid(f, f"fmt must be one of {sorted(FP6_FORMATS)}")
    wt, dt = _host_weight(w)
    Co, Ci = wt.shape
    if (l1 is None) != (l2 is None):
        _invalid(f, "give both factors or neither")
    rank = 0 if l1 is None else np.asarray(l1).shape[-1]
    if l1 is not None and np.asarray(l1).ndim != 2:
        _invalid(f, "l1 must be 2-D [Ci][rank]")
    l1c = None if l1 is None else _factor(f, "l1", l1, (Ci, rank))
    l2c = None if l2 is None else _factor(f, "l2", l2, (rank, Co))
    h = ctypes.c_void_p()
    _check(load().dq_prepare_weights_w6(_ptr(wt), dt, Ci, Co, rank, _ptr(l1c), _ptr(l2c), FP6_FORMATS[fmt], device,
                                        ctypes.byref(h)), f)
    wts = Weights(h)
    wts.fp6_format = fmt
    return wts


def dq_act6_create(w: Weights, N: int) -> Act6:
    h = ctypes.c_void_p()
    _check(load().dq_act6_create(w.handle, N, ctypes.byref(h)), "dq_act6_create")
    return Act6(h, w, N)


def dq_quantize_act6(w: Weights, x, a: Act6, stream=None):
    _check_pair("dq_quantize_act6", w, a)
    _check_x("dq_quantize_act6", w, a, x)
    _check(load().dq_quantize_act6(w.handle, _ptr(x), _dtype_of(x), a.handle, _stream(stream)), "dq_quantize_act6")


def dq_linear6_forward(w: Weights, a: Act6, y, stream=None):
    _check_pair("dq_linear6_forward", w, a)
    _check_y("dq_linear6_forward", w, a, y)
    _check(load().dq_linear6_forward(w.handle, a.handle, _ptr(y), _stream(stream)), "dq_linear6_forward")


def dq_linear6(w: Weights, x, a: Act6, y, stream=None):
    _check_pair("dq_linear6", w, a)
    _check_x("dq_linear6", w, a, x)
    _check_y("dq_linear6", w, a, y)
    _check(load().dq_linear6(w.handle, _ptr(x), _dtype_of(x), a.handle, _ptr(y), _stream(stream)), "dq_linear6")


def dq_act6_export(a: Act6, stream=None) -> dict:
    w = a.weights
    N, Ci, r = a.N, w.Ci, w.rank
    out = dict(codes=np.zeros((N, Ci // 4 * 3), np.uint8), scales=np.zeros((N, Ci // 32), np.uint8),
               U=np.zeros((N, r), np.uint16))
    _check(load().dq_act6_export(a.handle, _ptr(out["codes"]), _ptr(out["scales"]), _ptr(out["U"]), _stream(stream)),
           "dq_act6_export")
    return out


# -------------------------------------------------------- rotated-basis layers ----
class Orbit:
    """Owns a dq_orbit handle (a rotated, Lloyd-Max-coded weight)."""

    def __init__(self, handle, Ci, Co, wbits, abits, device):
        self.handle, self.Ci, self.Co, self.wbits, self.abits, self.device = handle, Ci, Co, wbits, abits, device
        self.rank = 0

    def __del__(self):
        if getattr(self, "handle", None) and _LIB is not None:
            _LIB.dq_orbit_destroy(self.handle)
            self.handle = None


class OrbitAct:
    """Owns a dq_orbit_act handle (keeps its weight alive)."""

    def __init__(self, handle, weights: Orbit, N: int):
        self.handle, self.weights, self.N = handle, weights, N

    def __del__(self):
        if getattr(self, "handle", None) and _LIB is not None:
            _LIB.dq_orbit_act_destroy(self.handle)
            self.handle = None


def dq_orbit_prepare(w, perm, wbits: int = 4, abits: int = 4, device: int = 0) -> Orbit:
    f = "dq_orbit_prepare"
    wt, dt = _host_weight(w)
    Co, Ci = wt.shape
    p = np.ascontiguousarray(np.asarray(perm), dtype=np.int32)
    if p.shape != (Ci,):
        _invalid(f, f"perm has shape {p.shape}; expected ({Ci},)")
    h = ctypes.c_void_p()
    _check(load().dq_orbit_prepare(_ptr(wt), dt, Ci, Co, _ptr(p), wbits, abits, device, ctypes.byref(h)), f)
    return Orbit(h, Ci, Co, wbits, abits, device)


def dq_orbit_export(o: Orbit) -> dict:
    out = dict(wlev=np.zeros(1 << o.wbits, np.uint16), alev=np.zeros(1 << o.abits, np.uint16),
               wcodes=np.zeros((o.Co, o.Ci // 2), np.uint8), wscale=np.zeros(o.Co, np.float32))
    _check(load().dq_orbit_export(o.handle, _ptr(out["wlev"]), _ptr(out["alev"]), _ptr(out["wcodes"]),
                                  _ptr(out["wscale"])), "dq_orbit_export")
    return out


def dq_orbit_act_create(o: Orbit, N: int) -> OrbitAct:
    h = ctypes.c_void_p()
    _check(load().dq_orbit_act_create(o.handle, N, ctypes.byref(h)), "dq_orbit_act_create")
    return OrbitAct(h, o, N)


def dq_orbit_quantize_act(o: Orbit, x, a: OrbitAct, stream=None):
    _check_pair("dq_orbit_quantize_act", o, a)
    _check_x("dq_orbit_quantize_act", o, a, x)
    _check(load().dq_orbit_quantize_act(o.handle, _ptr(x), _dtype_of(x), a.handle, _stream(stream)),
           "dq_orbit_quantize_act")


def dq_orbit_forward(o: Orbit, a: OrbitAct, y, stream=None):
    _check_pair("dq_orbit_forward", o, a)
    _check_y("dq_orbit_forward", o, a, y)
    _check(load().dq_orbit_forward(o.handle, a.handle, _ptr(y), _stream(stream)), "dq_orbit_forward")


def dq_orbit_linear(o: Orbit, x, a: OrbitAct, y, stream=None):
    _check_pair("dq_orbit_linear", o, a)
    _check_x("dq_orbit_linear", o, a, x)
    _check_y("dq_orbit_linear", o, a, y)
    _check(load().dq_orbit_linear(o.handle, _ptr(x), _dtype_of(x), a.handle, _ptr(y), _stream(stream)),
           "dq_orbit_linear")


def dq_orbit_act_export(a: OrbitAct, stream=None) -> dict:
    out = dict(codes=np.zeros((a.N, a.weights.Ci // 2), np.uint8), scale=np.zeros(a.N, np.float32))
    _check(load().dq_orbit_act_export(a.handle, _ptr(out["codes"]), _ptr(out["scale"]), _stream(stream)),
           "dq_orbit_act_export")
    return out
