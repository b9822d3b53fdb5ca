"""Python binding of the fused linear + Jensen-Shannon distillation loss
(``include/distill.h``): argument marshalling only; every step runs in the library's
kernels.

Source: "perf(distillation): skip dW/dB calculation when parameters are frozen",
Summary: the student head's weight and bias gradients are computed only when they are
requested (``dw`` / ``db`` not None); with nothing requested only the forward runs.
"""
from __future__ import annotations

import ctypes

import torch

from . import _check, _ptr, _stream, lib


def workspace_bytes(BT: int, H: int, Ht: int, V: int, chunk: int, dx: bool, dw: bool,
                    db: bool) -> int:
    return int(lib.fused_linear_jsd_workspace_bytes(BT, H, Ht, V, chunk, int(dx), int(dw),
                                                    int(db)))


def _ld(t, name):
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be a [rows, cols] tensor with contiguous rows")
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def fused_linear_jsd(xs, ws, xt, wt, bs=None, bt=None, beta: float = 0.5,
                     temperature: float = 1.0, chunk: int = 1024, *, dx=True, dw=True, db=True,
                     workspace=None, stream=None):
    """Loss (fp32 [1]) and student gradients of the fused linear JSD distillation loss.

    xs [BT, H], ws [V, H], xt [BT, Ht], wt [V, Ht], bs / bt [V] or None, all bf16.
    dx / dw / db: True allocates the gradient, a tensor receives it, None / False skips it
    (a frozen student weight: no dW product and no dW buffers).  db needs bs.
    Returns (loss, dx, dw, db)."""
    BT, H = xs.shape
    V, Ht = wt.shape
    for t, n in ((xs, "xs"), (ws, "ws"), (xt, "xt"), (wt, "wt")):
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{n} must be bf16")
    if ws.shape != (V, H) or xt.shape[0] != BT or (ws.stride(0) != H and V > 1):
        raise ValueError("shapes: xs [BT, H], ws [V, H] contiguous, xt [BT, Ht], wt [V, Ht]")
    if wt.stride(0) != Ht and V > 1:
        raise ValueError("wt must be contiguous")
    dev = xs.device
    if dx is True:
        dx = torch.empty(BT, H, dtype=torch.bfloat16, device=dev)
    if dw is True:
        dw = torch.empty(V, H, dtype=torch.float32, device=dev)
    if db is True:
        db = torch.empty(V, dtype=torch.float32, device=dev) if bs is not None else None
    dx = dx if dx is not False else None
    dw = dw if dw is not False else None
    db = db if db is not False else None
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    need = workspace_bytes(BT, H, Ht, V, chunk, dx is not None, dw is not None, db is not None)
    if need == 0:
        raise ValueError("sizes not supported (H, Ht multiples of 8; see include/distill.h)")
    if workspace is None:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    off = (-workspace.data_ptr()) % 256              # the library wants 256-byte alignment
    wsp = ctypes.c_void_p(workspace.data_ptr() + off)
    wsb = workspace.numel() * workspace.element_size() - off
    lddx = _ld(dx, "dx") if dx is not None else H
    _check(lib.fused_linear_jsd(_ptr(xs), _ld(xs, "xs"), _ptr(ws), _ptr(bs), _ptr(xt),
                                _ld(xt, "xt"), _ptr(wt), _ptr(bt), BT, H, Ht, V, beta,
                                temperature, chunk, _ptr(loss), _ptr(dx), lddx, _ptr(dw),
                                _ptr(db), wsp, wsb, _stream(stream)))
    return loss, dx, dw, db


__all__ = ["workspace_bytes", "fused_linear_jsd"]
