"""A seeded sweep of random problems through the launch planner, each checked against
the fp64 oracle on every row and, with its parameters frozen, for a dx bit-identical to
the trainable call's.

The draws cover the planner's decisions without naming them, in four strata taken in
turn: any width (log-uniform over 1..24576: narrow rows, each elements-per-lane choice);
wide rows of a multiple of 8 elements (16-byte accesses); tall inputs of 2048..12000 rows
(persistent workgroups); wide rows of any width (odd widths are not 16-byte aligned and
take element accesses).  M is otherwise log-uniform over 1..12000 (a few wide rows are
split over workgroups).  Every operation, every storage type pair, the Gemma offset, a
LayerNorm bias and a residual-output gradient are drawn at random.  Sizes stay within 8M
elements so the oracle takes a few seconds per case.
"""
import numpy as np
import pytest
import torch

import workloads
from tests import gpu_parity as gp

pytestmark = pytest.mark.gpu

OPS = ["rmsnorm", "layernorm", "fused_add_rmsnorm"]
TYPES = [("bf16", "bf16"), ("fp16", "fp16"), ("fp32", "fp32"), ("bf16", "fp32"), ("fp16", "fp32")]
MAX_N = 24576
MAX_ELEMS = 8 << 20


def _log_uniform(rng, lo, hi):
    return int(np.clip(round(np.exp(rng.uniform(np.log(lo), np.log(hi)))), lo, hi))


def _draws(n=96, seed=0x5EED):
    """Four strata in turn: any width; wide rows of a multiple of 8 elements (16-byte
    accesses); tall inputs; wide rows of any width."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = i % 4
        if kind == 0:
            N = _log_uniform(rng, 1, MAX_N)
        elif kind == 1:
            N = 8 * int(rng.integers(33, MAX_N // 8 + 1))
        elif kind == 2:
            N = _log_uniform(rng, 64, 4096)
            if rng.integers(2):
                N = max(8, N // 8 * 8)
        else:
            N = int(rng.integers(257, MAX_N + 1))
        M = int(rng.integers(2048, 12001)) if kind == 2 else _log_uniform(rng, 1, 12000)
        M = max(1, min(M, MAX_ELEMS // N))
        op = OPS[int(rng.integers(3))]
        io, wt = TYPES[int(rng.integers(len(TYPES)))]
        gemma = op != "layernorm" and bool(rng.integers(2))
        eps = float(rng.choice([1e-6, 1e-5]))
        out.append(workloads.small(op, M, N, io, wt, eps=eps, offset=1.0 if gemma else 0.0,
                                   weight="gemma" if gemma else "unit",
                                   bias=bool(rng.integers(2)), dres=bool(rng.integers(2)),
                                   seed=1000 + i))
    return out


CASES = _draws()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import __graft_entry__
    __graft_entry__.ensure_built()


@pytest.mark.parametrize("wl", CASES, ids=lambda c: c.name)
def test_random_problem(wl):
    print("[case] sweep", wl.name, f"eps={wl.eps} bias={wl.bias} dres={wl.dres}", flush=True)
    t = workloads.generate(wl)
    g = gp.run_gpu(wl, t)
    fails = gp.compare_all_rows(wl, g, t)
    assert not fails, "\n".join(fails)
    frozen = gp.run_gpu(wl, t, dw=False, db=False)
    bits = torch.int32 if wl.io == "fp32" else torch.int16
    assert torch.equal(g["dx"].view(bits), frozen["dx"].view(bits))


# ---- the same with padded rows ---------------------------------------------------------
# Every row tensor lives inside a wider allocation (row stride N + pad, pad 0..64) at a
# lead offset of 0..pad elements, so row pitch and base alignment vary independently; dx
# overwrites dy (the fused add: dres) half the time.

def _strided_draws(n=32, seed=0x57D):
    rng = np.random.default_rng(seed)
    base = _draws(n, seed)
    out = []
    for wl in base:
        M = max(1, min(wl.M, (4 << 20) // wl.N))
        w2 = workloads.small(wl.op, M, wl.N, wl.io, wl.wt, eps=wl.eps, offset=wl.offset,
                             weight=wl.weight, bias=wl.bias, dres=wl.dres, seed=wl.seed + 500)
        pad = int(rng.integers(0, 65))
        leads = [int(rng.integers(0, pad + 1)) for _ in range(4)]
        out.append((w2, pad, leads, bool(rng.integers(2))))
    return out


STRIDED = _strided_draws()


def _padded(src, pad, lead):
    M, N = src.shape
    big = torch.zeros(M, N + pad, dtype=src.dtype, device=gp.dev())
    v = big[:, lead:lead + N]
    v.copy_(src.to(gp.dev()))
    return v


def _run_padded(wl, t, pad, leads, inplace, trainable):
    import normalization_row_wise_amd as rn
    w = t["w"].to(gp.dev())
    x = _padded(t["x"], pad, leads[0])
    dy = _padded(t["dy"], pad, leads[1])
    dw = True if trainable else None
    out = {}
    if wl.op == "rmsnorm":
        out["y"], out["rstd"] = rn.rmsnorm_fwd(x, w, t["eps"], t["offset"])
        out["dx"], out["dw"] = rn.rmsnorm_bwd(dy, x, w, t["eps"], t["offset"],
                                              dx=dy if inplace else None, dw=dw)
    elif wl.op == "layernorm":
        b = t["b"].to(gp.dev()) if "b" in t else None
        out["y"], out["mean"], out["rstd"] = rn.layernorm_fwd(x, w, b, t["eps"])
        out["dx"], out["dw"], out["db"] = rn.layernorm_bwd(dy, x, w, t["eps"],
                                                           dx=dy if inplace else None, dw=dw,
                                                           db=True if trainable else None)
    else:
        res = _padded(t["residual"], pad, leads[2])
        out["y"], out["residual_out"], out["rstd"] = rn.fused_add_rmsnorm_fwd(
            x, res, w, t["eps"], t["offset"])
        dres = _padded(t["dres"], pad, leads[3]) if "dres" in t else None
        target = (dres if dres is not None else dy) if inplace else None
        out["dx"], out["dw"] = rn.fused_add_rmsnorm_bwd(dy, out["residual_out"], w, t["eps"],
                                                        t["offset"], dres, dx=target, dw=dw)
        if inplace:
            assert out["dx"].data_ptr() == target.data_ptr()
    if inplace and wl.op != "fused_add_rmsnorm":
        assert out["dx"].data_ptr() == dy.data_ptr()
    torch.cuda.synchronize()
    return {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in out.items()}


@pytest.mark.parametrize("case", STRIDED,
                         ids=lambda c: f"{c[0].name}_pad{c[1]}_lead{'-'.join(map(str, c[2]))}"
                                       f"{'_inplace' if c[3] else ''}")
def test_random_padded_problem(case):
    wl, pad, leads, inplace = case
    print("[case] padded sweep", wl.name, f"pad={pad} leads={leads} inplace={inplace}",
          flush=True)
    t = workloads.generate(wl)
    g = _run_padded(wl, t, pad, leads, inplace, trainable=True)
    fails = gp.compare_all_rows(wl, g, t)
    assert not fails, "\n".join(fails)
    frozen = _run_padded(wl, t, pad, leads, inplace, trainable=False)
    bits = torch.int32 if wl.io == "fp32" else torch.int16
    assert torch.equal(g["dx"].view(bits), frozen["dx"].view(bits))
