"""Pins of the distillation oracle (oracle/distill.py) against facts fixed outside it.

  * scipy's Jensen-Shannon distance: its square is the symmetric JSD (beta = 0.5);
  * the entropy form of the weighted JSD, H(M) - beta H(T) - (1 - beta) H(S), computed
    with scipy.stats.entropy (an identity, not the KL form the oracle writes out);
  * torch fp64 autograd of the loss (an independent derivative of the same definition);
  * central finite differences of the loss with respect to x_s, W_s and b_s;
  * invariants: identical student and teacher give zero loss and zero gradients; the
    loss is unchanged by adding a constant to a token's logits (so each gradient row
    sums to zero); 0 <= J <= the entropy of the mixture weights (ln 2 at beta = 0.5);
    J_beta(S, T) = J_(1-beta)(T, S); temperature tau equals logits divided by tau.
The checks run against the oracle (they must pass) and against copies with a planted
mistake (each must be caught by at least one check).
"""
from __future__ import annotations

import types

import numpy as np
import pytest
import torch
from scipy.spatial.distance import jensenshannon
from scipy.stats import entropy

import oracle.distill as od


def _impl(**over):
    ns = types.SimpleNamespace(jsd_rows=od.jsd_rows, fused_linear_jsd=od.fused_linear_jsd,
                               log_softmax=od.log_softmax)
    for k, v in over.items():
        setattr(ns, k, v)
    return ns


def _case(seed, bt=3, h=4, ht=5, v=6, scale=1.5):
    rng = np.random.default_rng(seed)
    return dict(xs=rng.standard_normal((bt, h)) * scale, ws=rng.standard_normal((v, h)),
                bs=rng.standard_normal(v) * 0.3, xt=rng.standard_normal((bt, ht)) * scale,
                wt=rng.standard_normal((v, ht)), bt=rng.standard_normal(v) * 0.3)


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))


def _softmax(z, tau):
    e = np.exp(z / tau - (z / tau).max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


# ---- checks ---------------------------------------------------------------------------

def check_symmetric_vs_scipy(impl):
    rng = np.random.default_rng(1)
    for tau in (1.0, 2.5):
        zs, zt = rng.standard_normal((5, 7)) * 2, rng.standard_normal((5, 7)) * 2
        j, _ = impl.jsd_rows(zs, zt, 0.5, tau)
        s, t = _softmax(zs, tau), _softmax(zt, tau)
        ref = np.array([jensenshannon(s[i], t[i]) ** 2 for i in range(5)])
        assert rel(j, ref) < 1e-12, ("scipy", tau)


def check_weighted_entropy_form(impl):
    rng = np.random.default_rng(2)
    for beta in (0.1, 0.3, 0.8):
        zs, zt = rng.standard_normal((4, 9)) * 1.7, rng.standard_normal((4, 9)) * 1.7
        j, _ = impl.jsd_rows(zs, zt, beta, 1.0)
        s, t = _softmax(zs, 1.0), _softmax(zt, 1.0)
        m = beta * t + (1 - beta) * s
        ref = np.array([entropy(m[i]) - beta * entropy(t[i]) - (1 - beta) * entropy(s[i])
                        for i in range(4)])
        assert rel(j, ref) < 1e-10, ("entropy form", beta)


def check_vs_torch_autograd(impl):
    for seed, beta, tau in ((3, 0.5, 1.0), (4, 0.25, 2.0), (5, 0.9, 0.7)):
        c = _case(seed)
        o = impl.fused_linear_jsd(c["xs"], c["ws"], c["bs"], c["xt"], c["wt"], c["bt"], beta, tau)
        xs, ws, bs = (torch.tensor(c[k], dtype=torch.float64, requires_grad=True)
                      for k in ("xs", "ws", "bs"))
        zt = torch.tensor(c["xt"] @ c["wt"].T + c["bt"], dtype=torch.float64)
        ls = torch.log_softmax((xs @ ws.T + bs) / tau, dim=1)
        lt = torch.log_softmax(zt / tau, dim=1)
        m = beta * lt.exp() + (1 - beta) * ls.exp()
        kl_t = (lt.exp() * (lt - m.log())).sum(1)
        kl_s = (ls.exp() * (ls - m.log())).sum(1)
        loss = (beta * kl_t + (1 - beta) * kl_s).mean()
        gx, gw, gb = torch.autograd.grad(loss, (xs, ws, bs))
        assert abs(o["loss"] - loss.item()) <= 1e-12 * max(1.0, abs(loss.item())), ("loss", seed)
        assert rel(o["dx"], gx) < 1e-10, ("dx", seed)
        assert rel(o["dw"], gw) < 1e-10, ("dw", seed)
        assert rel(o["db"], gb) < 1e-10, ("db", seed)


def check_finite_differences(impl):
    for seed, beta, tau in ((6, 0.5, 1.0), (7, 0.2, 2.5)):
        c = _case(seed, bt=2, h=3, ht=3, v=5)
        f = lambda cc: impl.fused_linear_jsd(cc["xs"], cc["ws"], cc["bs"], cc["xt"], cc["wt"],
                                             cc["bt"], beta, tau)["loss"]
        o = impl.fused_linear_jsd(c["xs"], c["ws"], c["bs"], c["xt"], c["wt"], c["bt"], beta, tau)
        for key, grad in (("xs", "dx"), ("ws", "dw"), ("bs", "db")):
            num = np.zeros_like(c[key])
            for idx in np.ndindex(c[key].shape):
                h = 1e-6 * max(1.0, abs(c[key][idx]))
                cp = {k: v.copy() for k, v in c.items()}
                cm = {k: v.copy() for k, v in c.items()}
                cp[key][idx] += h
                cm[key][idx] -= h
                num[idx] = (f(cp) - f(cm)) / (2 * h)
            assert rel(o[grad], num) < 1e-6, ("fd", key, seed)


def check_invariants(impl):
    c = _case(8, bt=4, h=5, ht=5, v=7)
    # identical heads: zero loss, zero gradients
    o = impl.fused_linear_jsd(c["xs"], c["ws"], c["bs"], c["xs"], c["ws"], c["bs"], 0.3, 1.3)
    assert abs(o["loss"]) < 1e-15 and np.abs(o["dx"]).max() < 1e-15
    assert np.abs(o["dw"]).max() < 1e-15 and np.abs(o["db"]).max() < 1e-15
    rng = np.random.default_rng(9)
    zs, zt = rng.standard_normal((6, 11)) * 3, rng.standard_normal((6, 11)) * 3
    for beta in (0.5, 0.15, 0.7):
        j, dz = impl.jsd_rows(zs, zt, beta, 1.0)
        bound = entropy([beta, 1 - beta])
        assert np.all(j >= -1e-15) and np.all(j <= bound + 1e-12), ("bound", beta)
        # a constant added to a token's logits changes nothing
        j2, dz2 = impl.jsd_rows(zs + 4.0, zt - 2.0, beta, 1.0)
        assert rel(j2, j) < 1e-12 and np.abs(dz.sum(axis=1)).max() < 1e-14 * np.abs(dz).max() * 11
        # J_beta(S, T) = J_(1-beta)(T, S)
        jr, _ = impl.jsd_rows(zt, zs, 1 - beta, 1.0)
        assert rel(jr, j) < 1e-12, ("swap", beta)
    # mixture weight 0 or 1: M is S or T itself, so J and its gradient vanish
    for beta in (0.0, 1.0):
        j, dz = impl.jsd_rows(zs, zt, beta, 1.0)
        assert np.abs(j).max() < 1e-14 and np.abs(dz).max() < 1e-14, ("end point", beta)
    # temperature: tau on the logits equals logits divided by tau
    for tau in (0.5, 3.0):
        jt, dzt = impl.jsd_rows(zs, zt, 0.4, tau)
        j1, dz1 = impl.jsd_rows(zs / tau, zt / tau, 0.4, 1.0)
        assert rel(jt, j1) < 1e-12 and rel(dzt, dz1 / tau) < 1e-12, ("tau", tau)


def check_frozen_skips_only_the_skipped(impl):
    c = _case(10)
    full = impl.fused_linear_jsd(c["xs"], c["ws"], c["bs"], c["xt"], c["wt"], c["bt"], 0.5, 1.0)
    part = impl.fused_linear_jsd(c["xs"], c["ws"], c["bs"], c["xt"], c["wt"], c["bt"], 0.5, 1.0,
                                 need_dw=False, need_db=False)
    assert part["dw"] is None and part["db"] is None
    assert np.array_equal(part["dx"], full["dx"]) and part["loss"] == full["loss"]


ALL_CHECKS = [check_symmetric_vs_scipy, check_weighted_entropy_form, check_vs_torch_autograd,
              check_finite_differences, check_invariants, check_frozen_skips_only_the_skipped]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_passes(check):
    check(_impl())


# ---- planted mistakes ---------------------------------------------------------------------

def _jsd_mutant(kind):
    def jsd_rows(zs, zt, beta, temperature):
        tau = float(temperature)
        b = float(beta)
        if kind == "no_tau_logits":
            tau_l = 1.0
        else:
            tau_l = tau
        ls = od.log_softmax(np.asarray(zs, np.float64) / tau_l)
        lt = od.log_softmax(np.asarray(zt, np.float64) / tau_l)
        s, t = np.exp(ls), np.exp(lt)
        m = (1 - b) * t + b * s if kind == "mixture_swapped" else b * t + (1 - b) * s
        lm = np.log(m)
        kl_t = (t * (lt - lm)).sum(axis=1)
        kl_s = (s * (ls - lm)).sum(axis=1)
        j = b * kl_t + (1 - b) * kl_s
        if kind == "kl_weights_swapped":
            j = (1 - b) * kl_t + b * kl_s
        g = (1 - b) * (ls - lm)
        if kind == "grad_from_teacher":
            g = b * (lt - lm)
        if kind == "no_projection":
            dz = s * g / tau
        else:
            dz = s * (g - (s * g).sum(axis=1, keepdims=True)) / tau
        if kind == "no_tau_grad":
            dz = dz * tau
        return j, dz
    return jsd_rows


def _fl_mutant(kind):
    def fused_linear_jsd(xs, ws, bs, xt, wt, bt, beta=0.5, temperature=1.0, need_dx=True,
                         need_dw=True, need_db=True):
        o = od.fused_linear_jsd(xs, ws, bs, xt, wt, bt, beta, temperature, need_dx, need_dw,
                                need_db)
        n = np.asarray(xs).shape[0]
        if kind == "sum_not_mean" and o["dx"] is not None:
            o["loss"] *= n
        if kind == "dw_uses_teacher_input" and o["dw"] is not None:
            o["dw"] = o["dz"].T @ np.asarray(xt, np.float64)[:, : np.asarray(xs).shape[1]]
        if kind == "student_bias_dropped":
            oo = od.fused_linear_jsd(xs, ws, None, xt, wt, bt, beta, temperature, need_dx,
                                     need_dw, False)
            oo["db"] = o["db"]
            o = oo
        if kind == "dx_uses_teacher_weight" and o["dx"] is not None:
            o["dx"] = o["dz"] @ np.asarray(wt, np.float64)[:, : np.asarray(xs).shape[1]]
        return o
    return fused_linear_jsd


def _fl_with(jsd):
    """fused_linear_jsd built on a (mutated) jsd_rows, the rest as the oracle."""
    def fused_linear_jsd(xs, ws, bs, xt, wt, bt, beta=0.5, temperature=1.0, need_dx=True,
                         need_dw=True, need_db=True):
        zs = np.asarray(xs) @ np.asarray(ws).T + (0 if bs is None else np.asarray(bs))
        zt = np.asarray(xt) @ np.asarray(wt).T + (0 if bt is None else np.asarray(bt))
        j, dj = jsd(zs, zt, beta, temperature)
        n = zs.shape[0]
        dz = dj / n
        return {"loss": j.sum() / n, "per_token": j, "zs": zs, "zt": zt, "dz": dz,
                "dx": dz @ np.asarray(ws) if need_dx else None,
                "dw": dz.T @ np.asarray(xs) if need_dw else None,
                "db": dz.sum(0) if (need_db and bs is not None) else None}
    return fused_linear_jsd


JSD_MUTANTS = ["no_tau_logits", "mixture_swapped", "kl_weights_swapped", "grad_from_teacher",
               "no_projection", "no_tau_grad"]
FL_MUTANTS = ["sum_not_mean", "dw_uses_teacher_input", "student_bias_dropped",
              "dx_uses_teacher_weight"]


@pytest.mark.parametrize("kind", JSD_MUTANTS + FL_MUTANTS)
def test_planted_mistake_is_caught(kind):
    if kind in JSD_MUTANTS:
        j = _jsd_mutant(kind)
        impl = _impl(jsd_rows=j, fused_linear_jsd=_fl_with(j))
    else:
        impl = _impl(fused_linear_jsd=_fl_mutant(kind))
    caught = []
    for check in ALL_CHECKS:
        try:
            check(impl)
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"no pin catches the planted mistake {kind}"


def test_zero_probability_terms():
    """Logits far apart: some probabilities underflow to 0; their terms count as 0."""
    zs = np.array([[0.0, -800.0, 1.0]])
    zt = np.array([[-800.0, 0.0, 1.0]])
    j, dz = od.jsd_rows(zs, zt, 0.5, 1.0)
    assert np.all(np.isfinite(j)) and np.all(np.isfinite(dz))
    assert 0.0 <= j[0] <= np.log(2.0)
