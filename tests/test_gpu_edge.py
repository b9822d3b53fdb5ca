"""GPU parity on the degenerate inputs of the method: rows with zero variance
(LayerNorm) or all zeros (RMSNorm), eps = 0, and magnitudes far from 1 (1e18 and 1e-18,
where the mean square leaves the range of the fp32 reciprocal-square-root estimate and
the kernels take the exact fp64 path).  Each row kind is mixed into one batch with
ordinary rows, so every launch shape sees it (the split-row kernels included: a few long
rows).

Each case prints what it is before touching the GPU.
"""
import numpy as np
import pytest
import torch

import workloads
from tests import gpu_parity as gp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import __graft_entry__
    __graft_entry__.ensure_built()


def _say(*a):
    print("[case]", *a, flush=True)


def _shaped(t, kind, io):
    """Rewrite some rows of x (and residual) in place: every 7th row constant, every
    11th all zeros, every 5th scaled by 1e18, every 13th by 1e-18."""
    td = workloads.TORCH_DTYPES[io]
    for key in ("x", "residual"):
        if key not in t:
            continue
        x = t[key].float()
        M = x.shape[0]
        if kind == "degenerate":
            x[0::7] = x[0::7, :1]            # constant rows: zero variance
            x[3::11] = 0.0                   # all-zero rows
            if key == "residual":
                x[3::11] = 0.0
        elif kind == "magnitude" and io != "fp16":
            x[1::5] *= 1e18
            x[2::13] *= 1e-18
        t[key] = x.to(td)
        assert M > 0
    return t


CASES = [
    # op, M, N, io, eps, kind
    ("layernorm", 300, 4096, "bf16", 1e-5, "degenerate"),
    ("layernorm", 300, 4096, "fp32", 1e-5, "degenerate"),
    ("layernorm", 1000, 128, "bf16", 1e-5, "degenerate"),
    ("rmsnorm", 300, 4096, "bf16", 1e-6, "degenerate"),
    ("rmsnorm", 1000, 128, "fp16", 1e-6, "degenerate"),
    ("fused_add_rmsnorm", 300, 8192, "bf16", 1e-6, "degenerate"),
    ("rmsnorm", 300, 4096, "bf16", 1e-6, "magnitude"),
    ("rmsnorm", 300, 4096, "fp32", 0.0, "magnitude"),
    ("layernorm", 300, 4096, "bf16", 0.0, "magnitude"),
    ("layernorm", 1000, 64, "fp32", 1e-5, "magnitude"),
    ("fused_add_rmsnorm", 300, 4096, "bf16", 1e-6, "magnitude"),
    # few long rows: the split-row kernels
    ("layernorm", 14, 8192, "bf16", 1e-5, "degenerate"),
    ("fused_add_rmsnorm", 14, 8192, "bf16", 1e-6, "degenerate"),
    ("rmsnorm", 14, 8192, "fp32", 0.0, "magnitude"),
    ("layernorm", 12, 8192, "bf16", 0.0, "magnitude"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_{c[1]}x{c[2]}_{c[3]}_eps{c[4]}_{c[5]}")
def test_degenerate_and_extreme_rows(case):
    op, M, N, io, eps, kind = case
    wl = workloads.small(op, M, N, io, eps=eps, offset=1.0 if op != "layernorm" else 0.0,
                         weight="gemma" if op != "layernorm" else "unit", seed=900 + M + N)
    _say(wl.name, kind)
    t = _shaped(workloads.generate(wl), kind, io)
    g = gp.run_gpu(wl, t)
    o = gp.run_oracle(wl, t)
    for k, v in o.items():
        if v is not None:
            assert np.all(np.isfinite(v)), f"oracle {k} not finite: the case is ill-posed"
    fails = gp.compare(wl, g, o)
    assert not fails, "\n".join(fails)
