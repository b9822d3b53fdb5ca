"""GPU parity of the narrow-row path: rows of at most 256 elements with 16-byte
accesses run teams of 8, 16 or 32 lanes, several rows per wave.  Compared with the
fp64 oracle element by element; rows counts are ragged and span many workgroup passes.

Each case prints what it is before touching the GPU.
"""
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


NARROW_N = [8, 16, 24, 64, 72, 96, 128, 136, 200, 256]
TYPES = [("bf16", "bf16"), ("fp16", "fp16"), ("fp32", "fp32"), ("bf16", "fp32"), ("fp16", "fp32")]
OPS = ["rmsnorm", "layernorm", "fused_add_rmsnorm"]
ROWS = [1, 5, 33, 1000, 4097]


def _cases():
    out = []
    for i, n in enumerate(NARROW_N):
        for j, (io, wt) in enumerate(TYPES):
            op = OPS[(i + j) % 3]
            m = ROWS[(i + 2 * j) % len(ROWS)]
            off = 1.0 if op != "layernorm" and (i + j) % 2 else 0.0
            out.append(workloads.small(op, m, n, io, wt, offset=off,
                                       weight="gemma" if off else "unit", seed=300 + 7 * i + j))
    return out


@pytest.mark.parametrize("wl", _cases(), ids=lambda c: c.name)
def test_narrow_rows(wl):
    _say(wl.name)
    fails = gp.check(wl)
    assert not fails, "\n".join(fails)


@pytest.mark.parametrize("wl", workloads.EXTRAS, ids=lambda c: c.name)
def test_narrow_named_workload(wl):
    _say(wl.name)
    fails = gp.check(wl)
    assert not fails, "\n".join(fails)


@pytest.mark.parametrize("op", OPS)
def test_narrow_frozen_dx_bit_identical(op):
    wl = workloads.small(op, 3001, 128, "bf16", offset=1.0 if op != "layernorm" else 0.0,
                         seed=77)
    _say("narrow frozen", wl.name)
    t = workloads.generate(wl)
    full = gp.run_gpu(wl, t, dw=True, db=True)
    frozen = gp.run_gpu(wl, t, dw=False, db=False)
    assert torch.equal(full["dx"].view(torch.int16), frozen["dx"].view(torch.int16))
    again = gp.run_gpu(wl, t, dw=True, db=True)
    assert torch.equal(again["dw"], full["dw"])


@pytest.mark.parametrize("n", [64, 128, 256])
def test_narrow_strided_inplace(n):
    import normalization_row_wise_amd as rn
    wl = workloads.small("rmsnorm", 517, n, "bf16", offset=1.0, weight="gemma", seed=n)
    _say("narrow strided+inplace", wl.name)
    t = workloads.generate(wl)
    o = gp.run_oracle(wl, t)
    M, N, pad = wl.M, n, 24

    def strided(src, lead):
        big = torch.zeros(M, N + pad, dtype=torch.bfloat16, device=gp.dev())
        v = big[:, lead:lead + N]
        v.copy_(src.to(gp.dev()))
        return v, big

    x, _ = strided(t["x"], 8)
    dy, _ = strided(t["dy"], 16)
    yv, ybig = strided(torch.full_like(t["x"], 3.0), 8)
    w = t["w"].to(gp.dev())
    y, _ = rn.rmsnorm_fwd(x, w, t["eps"], t["offset"], y=yv)
    dx, dw = rn.rmsnorm_bwd(dy, x, w, t["eps"], t["offset"], dx=dy)
    torch.cuda.synchronize()
    assert dx.data_ptr() == dy.data_ptr()
    for k, g in (("y", y), ("dx", dx)):
        rep = gp.io_report(g.cpu(), o[k], "bf16")
        assert gp.io_ok(rep, "bf16"), (k, rep)
    assert gp.f32_report(dw.cpu(), o["dw"]) <= gp.REL_GRAD
    # the padding around y is untouched
    assert torch.all(ybig[:, :8] == 0) and torch.all(ybig[:, 8 + N:] == 0)
