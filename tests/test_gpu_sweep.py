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
