"""fp64 CPU oracle: RMSNorm, LayerNorm and FusedAddRMSNorm, forward and backward.

TEST INFRASTRUCTURE. This module is the correctness oracle.  Only the test suite,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import it;
the HIP product path never imports, links or calls anything here, and nothing here
imports the product.

Every function is the plain definition written out in float64 with numpy, one row
at a time in the mathematical sense (vectorised over rows, no blocking, fusion or
reordering).  Inputs are the exact fp64 values of the stored bf16 / fp16 / fp32
tensors; ``eps`` and ``offset`` are the float32 values a kernel receives.  Outputs
stay in fp64: callers round them once with ``oracle.rounding.round_to``.

Sources (web pages, cited by title and section):
  [frozen]  "perf(norm): skip dW/dB calculation when parameters are frozen (#1067)"
  [gemma]   "fix(cutedsl): fuse Gemma RMSNorm weight offset in FP32"

The pages name the operations but never print their formulas.  The readings taken
here (textbook and torch.nn.functional conventions) are:
  * RMSNorm: rstd = 1/sqrt(mean_j x_j^2 + eps), eps inside the root, mean over N.
  * LayerNorm: biased variance (divide by N), eps inside the root.
  * Gemma offset ([gemma], Summary): the weight is used as (w + offset) with the sum
    formed exactly (here fp64; the page asks for at least FP32 instead of rounding the
    sum to the weight's 16-bit type).  LayerNorm takes no offset.
  * FusedAddRMSNorm: s = x + residual is rounded once to the I/O type; that rounded
    value is stored as residual_out and is what gets normalised ([gemma], PyTorch
    accuracy comparison: the backward works from the rounded saved residual).  The
    gradient treats the rounding as the identity, so d(x) = d(residual) =
    d(residual_out) + (RMSNorm backward at the rounded s).
  * dW / dB are sums over rows of dy * xhat and of dy ([frozen], Motivation and Key
    Changes describe them as reductions across tokens).
"""
from __future__ import annotations

import numpy as np

from .rounding import round_to

__all__ = [
    "rmsnorm_fwd", "rmsnorm_bwd",
    "layernorm_fwd", "layernorm_bwd",
    "fused_add_rmsnorm_fwd", "fused_add_rmsnorm_bwd",
    "rmsnorm_fwd_preadd_control",
]


def _rows(a) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64)
    if a.ndim != 2:
        raise ValueError("expected a [M, N] array")
    return a


def _vec(a, n) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64).reshape(-1)
    if a.shape[0] != n:
        raise ValueError("parameter length does not match N")
    return a


def rmsnorm_fwd(x, w, eps: float, offset: float = 0.0):
    """RMSNorm forward.  Returns (y, rstd).

    [gemma] Summary: the effective weight is w + offset, formed without rounding.
    """
    x = _rows(x)
    n = x.shape[1]
    weff = _vec(w, n) + float(offset)
    mean_sq = np.sum(x * x, axis=1) / n
    rstd = 1.0 / np.sqrt(mean_sq + float(eps))
    xhat = x * rstd[:, None]
    y = xhat * weff[None, :]
    return y, rstd


def rmsnorm_bwd(dy, x, w, eps: float, offset: float = 0.0):
    """RMSNorm backward.  Returns (dx, dw).

    With g = dy * (w + offset) and xhat = x * rstd:
        dx = rstd * (g - xhat * mean_j(g * xhat))
        dw = sum over rows of dy * xhat        (the offset is a constant: no effect on dw)
    The row statistics are recomputed from x here, never taken from a forward run.
    [frozen] Key Changes (RMSNorm backward with its dW accumulation);
    [gemma] Summary (the offset is applied inside the backward too).
    """
    x = _rows(x)
    dy = _rows(dy)
    n = x.shape[1]
    weff = _vec(w, n) + float(offset)
    _, rstd = rmsnorm_fwd(x, w, eps, offset)
    xhat = x * rstd[:, None]
    g = dy * weff[None, :]
    c = np.sum(g * xhat, axis=1) / n
    dx = rstd[:, None] * (g - xhat * c[:, None])
    dw = np.sum(dy * xhat, axis=0)
    return dx, dw


def layernorm_fwd(x, w, b, eps: float):
    """LayerNorm forward.  Returns (y, mean, rstd); ``b`` may be None (no bias).

    Two passes: mean first, then the biased variance of the centred row.
    [frozen] Key Changes (LayerNorm with weight and bias).
    """
    x = _rows(x)
    n = x.shape[1]
    w = _vec(w, n)
    mean = np.sum(x, axis=1) / n
    xc = x - mean[:, None]
    var = np.sum(xc * xc, axis=1) / n
    rstd = 1.0 / np.sqrt(var + float(eps))
    xhat = xc * rstd[:, None]
    y = xhat * w[None, :]
    if b is not None:
        y = y + _vec(b, n)[None, :]
    return y, mean, rstd


def layernorm_bwd(dy, x, w, eps: float):
    """LayerNorm backward.  Returns (dx, dw, db).

    With g = dy * w:
        dx = rstd * (g - mean_j(g) - xhat * mean_j(g * xhat))
        dw = sum over rows of dy * xhat,   db = sum over rows of dy
    [frozen] Key Changes (independent weight and bias gradients).
    """
    x = _rows(x)
    dy = _rows(dy)
    n = x.shape[1]
    w = _vec(w, n)
    _, mean, rstd = layernorm_fwd(x, w, None, eps)
    xhat = (x - mean[:, None]) * rstd[:, None]
    g = dy * w[None, :]
    c1 = np.sum(g, axis=1) / n
    c2 = np.sum(g * xhat, axis=1) / n
    dx = rstd[:, None] * (g - c1[:, None] - xhat * c2[:, None])
    dw = np.sum(dy * xhat, axis=0)
    db = np.sum(dy, axis=0)
    return dx, dw, db


def fused_add_rmsnorm_fwd(x, residual, w, eps: float, offset: float, io_dtype: str):
    """FusedAddRMSNorm forward.  Returns (y, residual_out, rstd).

    residual_out = round_io(x + residual); y = RMSNorm(residual_out) with w + offset.
    [gemma] Summary (Gemma offset on this op too) and PyTorch accuracy comparison
    (the rounded residual is what is saved).
    """
    s = _rows(x) + _rows(residual)          # exact: both operands are 16/32-bit values
    s_q = round_to(s, io_dtype)
    y, rstd = rmsnorm_fwd(s_q, w, eps, offset)
    return y, s_q, rstd


def fused_add_rmsnorm_bwd(dy, dres_out, residual_out, w, eps: float, offset: float):
    """FusedAddRMSNorm backward.  Returns (dx, dw); dx is also d(residual).

    dx = dres_out + RMSNorm backward evaluated at the saved (rounded) residual_out.
    ``dres_out`` may be None (no gradient reaches the residual output).
    [gemma] PyTorch accuracy comparison (residual-output gradient, rounded saved residual).
    """
    dx, dw = rmsnorm_bwd(dy, residual_out, w, eps, offset)
    if dres_out is not None:
        dx = dx + _rows(dres_out)
    return dx, dw


def rmsnorm_fwd_preadd_control(x, w, eps: float, offset: float, w_dtype: str):
    """The behaviour the Gemma fix removed: (w + offset) rounded to the weight's type
    before use.  A fixture for accuracy-magnitude checks, never a product path.
    [gemma] Summary (the old path added the offset to the 16-bit weight first).
    """
    n = _rows(x).shape[1]
    weff_rounded = round_to(_vec(w, n) + float(offset), w_dtype)
    return rmsnorm_fwd(x, weff_rounded, eps, 0.0)
