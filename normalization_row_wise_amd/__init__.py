"""Row-wise RMSNorm / LayerNorm / FusedAddRMSNorm for AMD MI355X (gfx950).

A thin ctypes binding over ``librownorm.so`` (C ABI in ``include/rownorm.h``).  The
functions keep the C names and only marshal arguments: torch supplies device memory
(outputs and the backward workspace are allocated with torch when not passed in) and
the current HIP stream; every step of the computation runs in the library's kernels.
There is no CPU fallback: a missing library raises at import time.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librownorm.so")

RN_F32, RN_F16, RN_BF16 = 0, 1, 2
RN_MAX_N = 24576
_DT = {torch.float32: RN_F32, torch.float16: RN_F16, torch.bfloat16: RN_BF16}

_vp, _i64, _f32, _i32, _sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int,
                              ctypes.c_size_t)

_SIGS = {
    "rn_bwd_workspace_bytes": (_sz, [_i64, _i64, _i32]),
    "rn_status_str": (ctypes.c_char_p, [_i32]),
    "rmsnorm_fwd": (_i32, [_vp, _i64, _vp, _vp, _i64, _vp, _i64, _i64, _f32, _f32, _i32, _i32, _vp]),
    "rmsnorm_bwd": (_i32, [_vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _sz, _i64, _i64, _f32,
                           _f32, _i32, _i32, _vp]),
    "rmsnorm_bwd_noalloc": (_i32, [_vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _i64, _i64, _f32,
                                   _f32, _i32, _i32, _vp]),
    "layernorm_fwd": (_i32, [_vp, _i64, _vp, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _f32, _i32, _i32,
                             _vp]),
    "layernorm_bwd": (_i32, [_vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _i64, _i64,
                             _f32, _i32, _i32, _vp]),
    "fused_add_rmsnorm_fwd": (_i32, [_vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _i64, _vp, _i64,
                                     _i64, _f32, _f32, _i32, _i32, _vp]),
    "fused_add_rmsnorm_bwd": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _vp,
                                     _sz, _i64, _i64, _f32, _f32, _i32, _i32, _vp]),
    # include/distill.h
    "fused_linear_jsd_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64, _i32, _i32, _i32]),
    "fused_linear_jsd": (_i32, [_vp, _i64, _vp, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64,
                                _f32, _f32, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
}


# Instrumentation (normalization_row_wise_amd/csrc/rn_instrument.h; not the product ABI).
_INSTRUMENT_SIGS = {"rn_set_timing_events": (_i32, [_i32, _vp, _vp])}


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library and declare its C signatures.  Raises if it is missing."""
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python normalization_row_wise_amd/build.py` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    for name, (res, args) in _INSTRUMENT_SIGS.items():   # optional
        f = getattr(lib, name, None)
        if f is not None:
            f.restype = res
            f.argtypes = args
    return lib


lib = load_library()


class RowNormError(RuntimeError):
    pass


def _check(status: int) -> None:
    if status != 0:
        raise RowNormError(f"rownorm status {status}: {lib.rn_status_str(status).decode()}")


def _ptr(t):
    """Device address of a tensor on the current GPU (the kernels would fault on a host
    address or on another device's memory, so anything else is refused here)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("every tensor argument must be a GPU tensor (got one on the CPU)")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"tensor on {t.device}, but the current device is "
                         f"cuda:{torch.cuda.current_device()}")
    return ctypes.c_void_p(t.data_ptr())


def _rows(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be [M, N]")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dt(t):
    try:
        return _DT[t.dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {t.dtype}") from None


def _opt(v, M, device):
    """True -> a new fp32 [M] tensor; None / False -> NULL; a tensor -> itself."""
    if v is True:
        return torch.empty(M, dtype=torch.float32, device=device)
    if v is None or v is False:
        return None
    return v


def workspace_bytes(M: int, N: int, n_param_grads: int) -> int:
    return int(lib.rn_bwd_workspace_bytes(M, N, n_param_grads))


def _workspace(ws, M, N, n, device):
    """Caller's workspace, or a torch allocation of the size the library asks for."""
    if ws is None:
        need = workspace_bytes(M, N, n) if n else 0
        if need == 0:
            return None, 0
        ws = new_workspace(need, device)
    return ws, ws.numel() * ws.element_size()


def new_workspace(nbytes: int, device=None):
    """A backward workspace of nbytes (device memory for the per-workgroup partial rows
    of dW / dB; its contents do not matter)."""
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _set_timing_events(kernel: int, start=None, stop=None) -> None:
    """Instrumentation for measurement harnesses: every launch of one kernel family made
    by this thread records its dispatch start / end into two torch.cuda.Events (kernel 0
    = forward, 1 = the backward's first kernel).  The events must have been recorded
    once (so that they exist).  None, None stops."""
    h = (lambda e: None if e is None else ctypes.c_void_p(e.cuda_event))
    _check(lib.rn_set_timing_events(kernel, h(start), h(stop)))


def rmsnorm_fwd(x, w, eps: float = 1e-6, offset: float = 0.0, *, y=None, rstd=True, stream=None):
    """y = x * rstd * (w + offset).  Returns (y, rstd); rstd=False skips the statistic."""
    M, N = x.shape
    ldx = _rows(x, "x")
    y = torch.empty_like(x, memory_format=torch.contiguous_format) if y is None else y
    rstd = _opt(rstd, M, x.device)
    _check(lib.rmsnorm_fwd(_ptr(x), ldx, _ptr(w), _ptr(y), _rows(y, "y"), _ptr(rstd), M, N, eps,
                           offset, _dt(x), _dt(w), _stream(stream)))
    return y, rstd


def rmsnorm_bwd(dy, x, w, eps: float = 1e-6, offset: float = 0.0, *, dx=None, dw=True,
                workspace=None, stream=None):
    """Returns (dx, dw).  dw=None (frozen weight) prunes the weight gradient."""
    M, N = x.shape
    dx = torch.empty_like(x, memory_format=torch.contiguous_format) if dx is None else dx
    if dw is True:
        dw = torch.empty(N, dtype=torch.float32, device=x.device)
    ws, wsb = _workspace(workspace, M, N, int(dw is not None), x.device)
    _check(lib.rmsnorm_bwd(_ptr(dy), _rows(dy, "dy"), _ptr(x), _rows(x, "x"), _ptr(w), _ptr(dx),
                           _rows(dx, "dx"), _ptr(dw), _ptr(ws), wsb, M, N, eps, offset, _dt(x),
                           _dt(w), _stream(stream)))
    return dx, dw


def rmsnorm_bwd_noalloc(dy, x, w, eps: float = 1e-6, offset: float = 0.0, *, dx=None, dw=True,
                        stream=None):
    """rmsnorm_bwd without a workspace: the library keeps the partial rows of dw in its
    own per-GPU scratch (8 MiB).  Returns (dx, dw)."""
    M, N = x.shape
    dx = torch.empty_like(x, memory_format=torch.contiguous_format) if dx is None else dx
    if dw is True:
        dw = torch.empty(N, dtype=torch.float32, device=x.device)
    _check(lib.rmsnorm_bwd_noalloc(_ptr(dy), _rows(dy, "dy"), _ptr(x), _rows(x, "x"), _ptr(w),
                                   _ptr(dx), _rows(dx, "dx"), _ptr(dw), M, N, eps, offset, _dt(x),
                                   _dt(w), _stream(stream)))
    return dx, dw


def layernorm_fwd(x, w, b=None, eps: float = 1e-5, *, y=None, mean=True, rstd=True, stream=None):
    """y = (x - mean) * rstd * w + b.  Returns (y, mean, rstd)."""
    M, N = x.shape
    y = torch.empty_like(x, memory_format=torch.contiguous_format) if y is None else y
    mean = _opt(mean, M, x.device)
    rstd = _opt(rstd, M, x.device)
    _check(lib.layernorm_fwd(_ptr(x), _rows(x, "x"), _ptr(w), _ptr(b), _ptr(y), _rows(y, "y"),
                             _ptr(mean), _ptr(rstd), M, N, eps, _dt(x), _dt(w), _stream(stream)))
    return y, mean, rstd


def layernorm_bwd(dy, x, w, eps: float = 1e-5, *, dx=None, dw=True, db=True, workspace=None,
                  stream=None):
    """Returns (dx, dw, db).  dw=None / db=None prune each parameter gradient."""
    M, N = x.shape
    dx = torch.empty_like(x, memory_format=torch.contiguous_format) if dx is None else dx
    if dw is True:
        dw = torch.empty(N, dtype=torch.float32, device=x.device)
    if db is True:
        db = torch.empty(N, dtype=torch.float32, device=x.device)
    n = int(dw is not None) + int(db is not None)
    ws, wsb = _workspace(workspace, M, N, n, x.device)
    _check(lib.layernorm_bwd(_ptr(dy), _rows(dy, "dy"), _ptr(x), _rows(x, "x"), _ptr(w), _ptr(dx),
                             _rows(dx, "dx"), _ptr(dw), _ptr(db), _ptr(ws), wsb, M, N, eps, _dt(x),
                             _dt(w), _stream(stream)))
    return dx, dw, db


def fused_add_rmsnorm_fwd(x, residual, w, eps: float = 1e-6, offset: float = 0.0, *, y=None,
                          residual_out=None, rstd=True, stream=None):
    """residual_out = round(x + residual); y = RMSNorm(residual_out).
    Returns (y, residual_out, rstd)."""
    M, N = x.shape
    y = torch.empty_like(x, memory_format=torch.contiguous_format) if y is None else y
    if residual_out is None:
        residual_out = torch.empty_like(x, memory_format=torch.contiguous_format)
    rstd = _opt(rstd, M, x.device)
    _check(lib.fused_add_rmsnorm_fwd(_ptr(x), _rows(x, "x"), _ptr(residual),
                                     _rows(residual, "residual"), _ptr(w), _ptr(y), _rows(y, "y"),
                                     _ptr(residual_out), _rows(residual_out, "residual_out"),
                                     _ptr(rstd), M, N, eps, offset, _dt(x), _dt(w),
                                     _stream(stream)))
    return y, residual_out, rstd


def fused_add_rmsnorm_bwd(dy, residual_out, w, eps: float = 1e-6, offset: float = 0.0,
                          dres_out=None, *, dx=None, dw=True, workspace=None, stream=None):
    """Returns (dx, dw); dx is the gradient of both x and residual."""
    M, N = residual_out.shape
    dx = torch.empty_like(dy, memory_format=torch.contiguous_format) if dx is None else dx
    if dw is True:
        dw = torch.empty(N, dtype=torch.float32, device=dy.device)
    ws, wsb = _workspace(workspace, M, N, int(dw is not None), dy.device)
    lddr = _rows(dres_out, "dres_out") if dres_out is not None else 0
    _check(lib.fused_add_rmsnorm_bwd(_ptr(dy), _rows(dy, "dy"), _ptr(dres_out), lddr,
                                     _ptr(residual_out), _rows(residual_out, "residual_out"),
                                     _ptr(w), _ptr(dx), _rows(dx, "dx"), _ptr(dw), _ptr(ws), wsb, M,
                                     N, eps, offset, _dt(dy), _dt(w), _stream(stream)))
    return dx, dw


__all__ = [
    "lib", "LIB_PATH", "RowNormError", "workspace_bytes", "new_workspace",
    "rmsnorm_fwd", "rmsnorm_bwd", "rmsnorm_bwd_noalloc", "layernorm_fwd", "layernorm_bwd",
    "fused_add_rmsnorm_fwd", "fused_add_rmsnorm_bwd",
]
