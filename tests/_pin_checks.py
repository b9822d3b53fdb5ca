"""Pin checks for the oracle, written against an implementation passed in.

Each ``check_*`` raises AssertionError when the implementation disagrees with a fact
fixed outside it: torch's fp64 CPU routines and autograd (an independent
implementation of the same definitions), central finite differences, closed-form
invariants of the gradients, and closed forms for constant rows.  The same checks
run against the real oracle (they must pass) and against copies of it with a planted
mistake (they must fail), so that every plausible slip is shown to be caught.
"""
from __future__ import annotations

import types

import numpy as np
import torch
import torch.nn.functional as F


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))


def _t(a, grad=False):
    return torch.tensor(np.asarray(a, np.float64), dtype=torch.float64, requires_grad=grad)


def _rng_case(seed, M, N):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, N)) * rng.uniform(0.5, 3.0)
    dy = rng.standard_normal((M, N))
    w = rng.standard_normal(N) * 0.3 + 0.7
    b = rng.standard_normal(N) * 0.2
    r = rng.standard_normal((M, N))
    ds = rng.standard_normal((M, N))
    return x, dy, w, b, r, ds


SHAPES = [(1, 1), (2, 3), (3, 7), (4, 16), (5, 64), (3, 257)]


def check_rmsnorm_vs_torch(impl: types.SimpleNamespace, tol=1e-12):
    for i, (M, N) in enumerate(SHAPES):
        x, dy, w, *_ = _rng_case(i, M, N)
        for eps, offset in ((1e-6, 0.0), (1e-2, 1.0), (0.5, -0.25)):
            y, rstd = impl.rmsnorm_fwd(x, w, eps, offset)
            dx, dw = impl.rmsnorm_bwd(dy, x, w, eps, offset)
            xt, wt = _t(x, True), _t(w, True)
            yt = F.rms_norm(xt, (N,), weight=wt + offset, eps=eps)
            gx, gw = torch.autograd.grad(yt, (xt, wt), _t(dy))
            ref_rstd = 1.0 / torch.sqrt(xt.detach().pow(2).mean(-1) + eps)
            assert rel(y, yt.detach()) < tol, ("rms y", M, N, eps, offset)
            assert rel(rstd, ref_rstd) < tol, ("rms rstd", M, N)
            assert rel(dx, gx) < tol, ("rms dx", M, N, eps, offset)
            assert rel(dw, gw) < tol, ("rms dw", M, N, eps, offset)


def check_layernorm_vs_torch(impl, tol=1e-12):
    for i, (M, N) in enumerate(SHAPES):
        x, dy, w, b, *_ = _rng_case(100 + i, M, N)
        for eps in (1e-5, 0.3):
            for bias in (b, None):
                y, mean, rstd = impl.layernorm_fwd(x, w, bias, eps)
                xt, wt = _t(x, True), _t(w, True)
                bt = _t(bias, True) if bias is not None else None
                yt = F.layer_norm(xt, (N,), wt, bt, eps)
                assert rel(y, yt.detach()) < tol, ("ln y", M, N, eps)
                assert rel(mean, xt.detach().mean(-1)) < tol, ("ln mean", M, N)
                ref_rstd = 1 / torch.sqrt(xt.detach().var(-1, unbiased=False) + eps)
                assert rel(rstd, ref_rstd) < tol, ("ln rstd", M, N)
            dx, dw, db = impl.layernorm_bwd(dy, x, w, eps)
            xt, wt, bt = _t(x, True), _t(w, True), _t(b, True)
            yt = F.layer_norm(xt, (N,), wt, bt, eps)
            gx, gw, gb = torch.autograd.grad(yt, (xt, wt, bt), _t(dy))
            # N = 1: the exact dx is zero (torch's fused kernel leaves ~1e-14 noise)
            if N == 1:
                assert np.all(dx == 0.0) and float(gx.abs().max()) < 1e-12
            else:
                assert rel(dx, gx) < tol, ("ln dx", M, N, eps)
            assert rel(dw, gw) < tol or np.abs(np.asarray(dw) - gw.numpy()).max() < 1e-12, ("ln dw", M, N)
            assert rel(db, gb) < tol, ("ln db", M, N)


def check_fused_add_vs_torch(impl, tol=1e-12):
    """FusedAddRMSNorm against a torch graph: s = x + r, its stored value rounded to
    the I/O type by torch's own cast (exact sum in fp32, then one cast), gradients
    passing straight through the rounding."""
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
    for i, (M, N) in enumerate(SHAPES):
        for io in ("bf16", "fp16", "fp32"):
            x, dy, w, _, r, ds = _rng_case(200 + i, M, N)
            # inputs are stored values of the I/O type
            x = torch.tensor(x, dtype=torch.float32).to(tdt[io]).double().numpy()
            r = torch.tensor(r, dtype=torch.float32).to(tdt[io]).double().numpy()
            eps, offset = 1e-6, 1.0
            y, s_q, rstd = impl.fused_add_rmsnorm_fwd(x, r, w, eps, offset, io)
            # torch: x + r of two 16/32-bit values is exact in fp32 unless the
            # exponents are > 16 apart; a rounding there still lands on the same
            # 16-bit value (the small term is below half a 16-bit spacing)
            s32 = torch.tensor(x, dtype=torch.float32) + torch.tensor(r, dtype=torch.float32)
            s_ref = s32.to(tdt[io]).double() if io != "fp32" else (
                torch.tensor(x) + torch.tensor(r)).float().double()
            assert np.array_equal(s_q, s_ref.numpy()), ("fused s_q", M, N, io)
            xt, rt, wt = _t(x, True), _t(r, True), _t(w, True)
            s = xt + rt
            s_st = s + (_t(s_q) - s).detach()           # value s_q, gradient identity
            yt = F.rms_norm(s_st, (N,), weight=wt + offset, eps=eps)
            loss = (yt * _t(dy)).sum() + (s_st * _t(ds)).sum()
            gx, gr, gw = torch.autograd.grad(loss, (xt, rt, wt))
            assert rel(y, yt.detach()) < tol, ("fused y", M, N, io)
            dx, dw = impl.fused_add_rmsnorm_bwd(dy, ds, s_q, w, eps, offset)
            assert rel(dx, gx) < tol and rel(dx, gr) < tol, ("fused dx", M, N, io)
            assert rel(dw, gw) < tol, ("fused dw", M, N, io)
            dx0, _ = impl.fused_add_rmsnorm_bwd(dy, None, s_q, w, eps, offset)
            assert rel(dx0 + ds, dx) < tol, ("fused dres optional", M, N, io)


def _fd(f, a, h_rel=1e-6):
    g = np.zeros_like(a)
    it = np.nditer(a, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        h = h_rel * max(1.0, abs(a[idx]))
        ap, am = a.copy(), a.copy()
        ap[idx] += h
        am[idx] -= h
        g[idx] = (f(ap) - f(am)) / (2 * h)
    return g


def check_finite_differences(impl, tol=1e-6):
    """Central differences of L = sum(dy * y) (+ sum(ds * s) for the fused add)."""
    for M in (1, 3):
        for N in (1, 2, 3, 7, 16):
            x, dy, w, b, r, ds = _rng_case(300 + 10 * M + N, M, N)
            eps, off = 1e-3, 0.5

            def lr_x(xx):
                return float(np.sum(dy * impl.rmsnorm_fwd(xx, w, eps, off)[0]))

            def lr_w(ww):
                return float(np.sum(dy * impl.rmsnorm_fwd(x, ww, eps, off)[0]))

            dx, dw = impl.rmsnorm_bwd(dy, x, w, eps, off)
            assert np.allclose(dx, _fd(lr_x, x), rtol=tol, atol=tol), ("fd rms dx", M, N)
            assert np.allclose(dw, _fd(lr_w, w), rtol=tol, atol=tol), ("fd rms dw", M, N)

            def ll(xx, ww, bb):
                return float(np.sum(dy * impl.layernorm_fwd(xx, ww, bb, eps)[0]))

            dx, dw, db = impl.layernorm_bwd(dy, x, w, eps)
            assert np.allclose(dx, _fd(lambda v: ll(v, w, b), x), rtol=tol, atol=tol), ("fd ln dx", M, N)
            assert np.allclose(dw, _fd(lambda v: ll(x, v, b), w), rtol=tol, atol=tol), ("fd ln dw", M, N)
            assert np.allclose(db, _fd(lambda v: ll(x, w, v), b), rtol=tol, atol=tol), ("fd ln db", M, N)

            # fused add without rounding (the I/O type is set aside: s = x + r exactly)
            def lf(xx, rr, ww):
                s = xx + rr
                return float(np.sum(dy * impl.rmsnorm_fwd(s, ww, eps, off)[0]) + np.sum(ds * s))

            dxf, dwf = impl.fused_add_rmsnorm_bwd(dy, ds, x + r, w, eps, off)
            assert np.allclose(dxf, _fd(lambda v: lf(v, r, w), x), rtol=tol, atol=tol), ("fd fa dx", M, N)
            assert np.allclose(dxf, _fd(lambda v: lf(x, v, w), r), rtol=tol, atol=tol), ("fd fa dr", M, N)
            assert np.allclose(dwf, _fd(lambda v: lf(x, r, v), w), rtol=tol, atol=tol), ("fd fa dw", M, N)


def check_invariants(impl):
    """Sums of the input gradient fixed by the algebra of the two norms.

    RMSNorm:   sum_j dx_j * xhat_j = rstd * eps / (ms + eps) * sum_j g_j * xhat_j
    LayerNorm: sum_j dx_j = 0 for any eps, and
               sum_j dx_j * xhat_j = rstd * eps / (var + eps) * sum_j g_j * xhat_j
    Both right-hand sides vanish at eps = 0.
    """
    rng = np.random.default_rng(11)
    for N in (2, 16, 1000):
        x = rng.standard_normal((4, N)) * 2 + 0.5
        dy = rng.standard_normal((4, N))
        w = rng.standard_normal(N)
        for eps in (0.0, 1e-6, 0.7):
            # RMSNorm
            off = 0.3
            _, rstd = impl.rmsnorm_fwd(x, w, eps, off)
            dx, _ = impl.rmsnorm_bwd(dy, x, w, eps, off)
            ms = np.mean(x * x, axis=1)
            xhat = x * rstd[:, None]
            g = dy * (w + off)
            lhs = np.sum(dx * xhat, axis=1)
            rhs = rstd * eps / (ms + eps) * np.sum(g * xhat, axis=1)
            scale = np.sum(np.abs(g * xhat), axis=1) * rstd
            assert np.all(np.abs(lhs - rhs) <= 1e-12 * scale), ("rms invariant", N, eps)
            # LayerNorm
            _, mean, rstd = impl.layernorm_fwd(x, w, None, eps)
            dx, _, _ = impl.layernorm_bwd(dy, x, w, eps)
            xc = x - np.mean(x, axis=1, keepdims=True)
            var = np.mean(xc * xc, axis=1)
            xhat = xc / np.sqrt(var + eps)[:, None]
            g = dy * w
            scale = np.sum(np.abs(g), axis=1) * rstd * (1 + np.max(np.abs(xhat), axis=1))
            assert np.all(np.abs(np.sum(dx, axis=1)) <= 1e-12 * scale), ("ln sum dx", N, eps)
            lhs = np.sum(dx * xhat, axis=1)
            rhs = rstd * eps / (var + eps) * np.sum(g * xhat, axis=1)
            assert np.all(np.abs(lhs - rhs) <= 1e-12 * scale * np.max(np.abs(xhat))), ("ln invariant", N, eps)


def check_closed_forms(impl):
    """Constant rows and pure standardisation."""
    N = 37
    w = np.linspace(-1.0, 2.0, N)
    b = np.linspace(0.5, -0.5, N)
    dy = np.cos(np.arange(3 * N).reshape(3, N))
    for c in (0.0, 1.5, -4.0):
        x = np.full((3, N), c)
        eps = 1e-3
        y, rstd = impl.rmsnorm_fwd(x, w, eps, 1.0)
        r = 1.0 / np.sqrt(c * c + eps)
        assert np.allclose(rstd, r, rtol=1e-14)
        assert np.allclose(y, c * r * (w + 1.0)[None, :], rtol=1e-14, atol=1e-300)
        y, mean, rstd = impl.layernorm_fwd(x, w, b, eps)
        assert np.allclose(mean, c, rtol=1e-14, atol=0)
        assert np.allclose(rstd, 1 / np.sqrt(eps), rtol=1e-14)
        assert np.allclose(y, np.broadcast_to(b, y.shape), rtol=0, atol=1e-15)
        dx, dw, db = impl.layernorm_bwd(dy, x, w, eps)
        g = dy * w
        assert np.allclose(dx, (g - g.mean(axis=1, keepdims=True)) / np.sqrt(eps), rtol=1e-12, atol=1e-12)
        assert np.allclose(dw, 0.0, atol=1e-12)
        assert np.allclose(db, dy.sum(axis=0), rtol=1e-14)
    # N = 1 LayerNorm: the centred value is 0, so y = b and dx = 0
    x = np.array([[3.0], [-2.0]])
    y, _, _ = impl.layernorm_fwd(x, [2.0], [0.25], 1e-5)
    assert np.all(y == 0.25)
    dx, _, _ = impl.layernorm_bwd(np.array([[1.0], [-1.0]]), x, [2.0], 1e-5)
    assert np.all(dx == 0.0)
    # unit weight, zero bias, eps -> 0: rows come out with mean 0 and mean square 1
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 500)) * 3 + 7
    y, _, _ = impl.layernorm_fwd(x, np.ones(500), np.zeros(500), 0.0)
    assert np.allclose(y.mean(axis=1), 0, atol=1e-12)
    assert np.allclose((y * y).mean(axis=1), 1, rtol=1e-12)
    y, _ = impl.rmsnorm_fwd(x, np.ones(500), 0.0, 0.0)
    assert np.allclose((y * y).mean(axis=1), 1, rtol=1e-12)


ALL_CHECKS = [
    check_rmsnorm_vs_torch,
    check_layernorm_vs_torch,
    check_fused_add_vs_torch,
    check_finite_differences,
    check_invariants,
    check_closed_forms,
]
