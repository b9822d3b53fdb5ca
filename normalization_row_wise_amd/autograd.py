"""torch.autograd functions and nn.Modules over the library's C-ABI calls.

Argument marshalling only: the forward and backward of every function are the
library's kernels.  A parameter that does not require a gradient reaches the backward
as a NULL gradient pointer, which selects the kernel instances without the dW / dB
reduction ("perf(norm): skip dW/dB calculation when parameters are frozen (#1067)",
Description and Key Changes: the per-parameter needs_input_grad flags decide what is
computed).  Gradients of the parameters are accumulated in fp32 and returned in the
parameter's dtype.

Inputs may have any leading shape; the last dimension is the normalised one.  The
backward recomputes the row statistics from the saved input, so nothing but the input
and the parameters is saved.
"""
from __future__ import annotations

import torch

from . import (fused_add_rmsnorm_bwd, fused_add_rmsnorm_fwd, layernorm_bwd, layernorm_fwd,
               rmsnorm_bwd, rmsnorm_fwd)


def _rows(t: torch.Tensor) -> torch.Tensor:
    """[..., N] as [M, N] with a contiguous last dimension and rows that do not overlap
    (a view when possible; an incoming gradient broadcast along rows is copied)."""
    t2 = t.reshape(-1, t.shape[-1])
    if (t2.shape[1] > 1 and t2.stride(1) != 1) or (t2.shape[0] > 1 and t2.stride(0) < t2.shape[1]):
        t2 = t2.contiguous()
    return t2


def _cast(g, like):
    return None if g is None else g.to(like.dtype)


def _check_casting(mode):
    """"gemma" is the one casting mode the pages describe ("fix(cutedsl): fuse Gemma RMSNorm
    weight offset in FP32", Summary): the offset is added to the weight in fp32 and every
    output is rounded once.  It is the library's only arithmetic policy."""
    if mode != "gemma":
        raise ValueError(f"casting_mode {mode!r} is not implemented (only 'gemma')")


class RMSNormFunction(torch.autograd.Function):
    """y = x * rstd * (w + offset); offset is added to w in fp32 inside the kernels
    ("fix(cutedsl): fuse Gemma RMSNorm weight offset in FP32", Summary).

    The trailing arguments follow the call in that page's reproduction
    (x, w, eps, offset, casting_mode, in_place, row_mode): casting_mode must be "gemma";
    in_place=True writes dx over the incoming gradient's storage; row_mode is accepted
    and ignored (the library picks the launch shape for the row width and count)."""

    @staticmethod
    def forward(ctx, x, weight, eps: float = 1e-6, offset: float = 0.0,
                casting_mode: str = "gemma", in_place: bool = False, row_mode=None):
        _check_casting(casting_mode)
        x2 = _rows(x)
        y, _ = rmsnorm_fwd(x2, weight, eps, offset, rstd=False)
        ctx.save_for_backward(x2, weight)
        ctx.eps, ctx.offset, ctx.shape, ctx.in_place = eps, offset, x.shape, in_place
        return y.view(x.shape)

    @staticmethod
    def backward(ctx, dy):
        x2, w = ctx.saved_tensors
        dy2 = _rows(dy)
        dx, dw = rmsnorm_bwd(dy2, x2, w, ctx.eps, ctx.offset, dx=dy2 if ctx.in_place else None,
                             dw=True if ctx.needs_input_grad[1] else None)
        return dx.view(ctx.shape), _cast(dw, w), None, None, None, None, None


class LayerNormFunction(torch.autograd.Function):
    """y = (x - mean) * rstd * w + b (b may be None)."""

    @staticmethod
    def forward(ctx, x, weight, bias=None, eps: float = 1e-5):
        x2 = _rows(x)
        y, _, _ = layernorm_fwd(x2, weight, bias, eps, mean=False, rstd=False)
        ctx.save_for_backward(x2, weight)
        ctx.eps, ctx.shape, ctx.has_bias = eps, x.shape, bias is not None
        return y.view(x.shape)

    @staticmethod
    def backward(ctx, dy):
        x2, w = ctx.saved_tensors
        need_b = ctx.has_bias and ctx.needs_input_grad[2]
        dx, dw, db = layernorm_bwd(_rows(dy), x2, w, ctx.eps,
                                   dw=True if ctx.needs_input_grad[1] else None,
                                   db=True if need_b else None)
        return dx.view(ctx.shape), _cast(dw, w), _cast(db, w), None


class FusedAddRMSNormFunction(torch.autograd.Function):
    """residual_out = round(x + residual); y = RMSNorm(residual_out).  Returns
    (y, residual_out); the gradient reaching residual_out is added to dx inside the
    backward kernel, and dx is the gradient of both x and residual.  casting_mode,
    in_place and row_mode as for RMSNormFunction (in place: dx over dy's storage)."""

    @staticmethod
    def forward(ctx, x, residual, weight, eps: float = 1e-6, offset: float = 0.0,
                casting_mode: str = "gemma", in_place: bool = False, row_mode=None):
        _check_casting(casting_mode)
        x2, r2 = _rows(x), _rows(residual)
        y, ro, _ = fused_add_rmsnorm_fwd(x2, r2, weight, eps, offset, rstd=False)
        ctx.save_for_backward(ro, weight)
        ctx.eps, ctx.offset, ctx.shape, ctx.in_place = eps, offset, x.shape, in_place
        return y.view(x.shape), ro.view(x.shape)

    @staticmethod
    def backward(ctx, dy, dres_out):
        ro, w = ctx.saved_tensors
        if dy is None:
            dy = torch.zeros(ctx.shape, dtype=ro.dtype, device=ro.device)
        dy2 = _rows(dy)
        dres = None if dres_out is None else _rows(dres_out)
        dx, dw = fused_add_rmsnorm_bwd(dy2, ro, w, ctx.eps, ctx.offset, dres,
                                       dx=dy2 if ctx.in_place else None,
                                       dw=True if ctx.needs_input_grad[2] else None)
        dx = dx.view(ctx.shape)
        return dx, dx, _cast(dw, w), None, None, None, None, None


class RMSNorm(torch.nn.Module):
    """RMSNorm over the last dimension.  offset = 1.0 with a zero-initialised weight is
    the Gemma convention (the weight stores w - 1)."""

    def __init__(self, n: int, eps: float = 1e-6, offset: float = 0.0, device=None,
                 dtype=torch.bfloat16):
        super().__init__()
        init = torch.zeros if offset else torch.ones
        self.weight = torch.nn.Parameter(init(n, device=device, dtype=dtype))
        self.eps, self.offset = eps, offset

    def forward(self, x):
        return RMSNormFunction.apply(x, self.weight, self.eps, self.offset)


class LayerNorm(torch.nn.Module):
    def __init__(self, n: int, eps: float = 1e-5, bias: bool = True, device=None,
                 dtype=torch.bfloat16):
        super().__init__()
        self.weight = torch.nn.Parameter(torch.ones(n, device=device, dtype=dtype))
        self.bias = torch.nn.Parameter(torch.zeros(n, device=device, dtype=dtype)) if bias else None
        self.eps = eps

    def forward(self, x):
        return LayerNormFunction.apply(x, self.weight, self.bias, self.eps)


class FusedAddRMSNorm(torch.nn.Module):
    """forward(x, residual) -> (y, residual_out)."""

    def __init__(self, n: int, eps: float = 1e-6, offset: float = 0.0, device=None,
                 dtype=torch.bfloat16):
        super().__init__()
        init = torch.zeros if offset else torch.ones
        self.weight = torch.nn.Parameter(init(n, device=device, dtype=dtype))
        self.eps, self.offset = eps, offset

    def forward(self, x, residual):
        return FusedAddRMSNormFunction.apply(x, residual, self.weight, self.eps, self.offset)


__all__ = ["RMSNormFunction", "LayerNormFunction", "FusedAddRMSNormFunction", "RMSNorm",
           "LayerNorm", "FusedAddRMSNorm"]
