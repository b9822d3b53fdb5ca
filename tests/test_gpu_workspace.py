"""GPU tests of the two-stage dW / dB reduction and its workspace.

The trainable backward writes one fp32 partial row of dW (and dB) per workgroup into
the caller's workspace and a second kernel sums them in a fixed order ("perf(norm): skip
dW/dB calculation when parameters are frozen (#1067)", Motivation: per-program partial
rows, then a sum over them).  These tests hold the results to the oracle's gates across
the launch shapes that produce many partial rows, reuse one workspace across shapes,
and check that the workspace's previous contents (zeros, NaNs, another call's partial
rows) never change a bit of the result.
"""
import ctypes

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
    import normalization_row_wise_amd as rn
    return rn


def _say(*a):
    print("[case]", *a, flush=True)


def _bwd(rn, wl, d, ws, dw=True, db=True):
    """One backward call with an explicit workspace; returns (dx, dw, db)."""
    N = wl.N
    dev = gp.dev()
    gw = torch.empty(N, dtype=torch.float32, device=dev) if dw else None
    gb = torch.empty(N, dtype=torch.float32, device=dev) if (db and wl.op == "layernorm") else None
    if wl.op == "rmsnorm":
        dx, _ = rn.rmsnorm_bwd(d["dy"], d["x"], d["w"], d["eps"], d["offset"], dw=gw,
                               workspace=ws)
    elif wl.op == "layernorm":
        dx, _, _ = rn.layernorm_bwd(d["dy"], d["x"], d["w"], d["eps"], dw=gw, db=gb,
                                    workspace=ws)
    else:
        _, ro, _ = rn.fused_add_rmsnorm_fwd(d["x"], d["residual"], d["w"], d["eps"], d["offset"])
        dx, _ = rn.fused_add_rmsnorm_bwd(d["dy"], ro, d["w"], d["eps"], d["offset"], d.get("dres"),
                                         dw=gw, workspace=ws)
    return dx, gw, gb


def _ngrads(wl, dw=True, db=True):
    return int(dw) + int(db and wl.op == "layernorm")


# Shapes whose trainable backward runs the row kernels with many partial rows, across
# the launch shapes: 512-thread workgroups of several teams, 256-thread workgroups
# (RMSNorm from 2048 rows), narrow teams (up to 512 partial rows), element accesses
# (N odd), wide rows at V = 48 (LDS blocks of stride 384, dW in LDS and dB in
# registers), fp32 and mixed weights, partial-row counts that are not multiples of the
# column sum's 32 slices and column counts that leave its last workgroup short.
CASES = [
    workloads.small("rmsnorm", 2048, 4096, "bf16", seed=201),
    workloads.small("rmsnorm", 4100, 4096, "bf16", offset=1.0, weight="gemma", seed=202),
    workloads.small("layernorm", 2048, 4096, "bf16", seed=203),
    workloads.small("layernorm", 777, 3001, "fp32", seed=204),
    workloads.small("fused_add_rmsnorm", 2048, 8192, "bf16", offset=1.0, weight="gemma", seed=205),
    workloads.small("fused_add_rmsnorm", 1000, 1000, "fp16", "fp32", seed=206),
    workloads.small("rmsnorm", 60000, 128, "bf16", seed=207),
    workloads.small("layernorm", 9000, 64, "bf16", seed=208),
    workloads.small("layernorm", 700, 18432, "bf16", seed=209),
    workloads.small("layernorm", 257, 20480, "fp16", seed=210),
    workloads.small("rmsnorm", 300, 24576, "bf16", "fp32", seed=211),
    workloads.small("rmsnorm", 333, 4097, "bf16", seed=212),
]


@pytest.mark.parametrize("wl", CASES, ids=lambda c: c.name)
def test_partial_rows_and_column_sum_match_oracle(wl):
    import normalization_row_wise_amd as rn
    _say("two-stage reduction", wl.name)
    t = workloads.generate(wl)
    d = gp.to_device(t)
    need = rn.workspace_bytes(wl.M, wl.N, _ngrads(wl))
    ws = torch.zeros(need, dtype=torch.uint8, device=gp.dev())
    dx, gw, gb = _bwd(rn, wl, d, ws)
    torch.cuda.synchronize()
    o = gp.run_oracle(wl, t)
    rep = gp.io_report(dx.cpu(), o["dx"], wl.io)
    assert gp.io_ok(rep, wl.io), rep
    assert gp.f32_report(gw.cpu(), o["dw"]) <= gp.REL_GRAD
    if gb is not None:
        assert gp.f32_report(gb.cpu(), o["db"]) <= gp.REL_GRAD
    # the same workspace again (holding the first call's partial rows), a fresh one full
    # of NaNs, and the frozen call: identical bits
    dx2, gw2, gb2 = _bwd(rn, wl, d, ws)
    nan_ws = torch.full((need // 4,), float("nan"), device=gp.dev()).view(torch.uint8)
    dx3, gw3, gb3 = _bwd(rn, wl, d, nan_ws)
    dxf, _, _ = _bwd(rn, wl, d, None, dw=False, db=False)
    torch.cuda.synchronize()
    bits = gp._BITS_VIEW[wl.io]
    for a in (dx2, dx3, dxf):
        assert torch.equal(a.view(bits), dx.view(bits))
    assert torch.equal(gw2, gw) and torch.equal(gw3, gw)
    if gb is not None:
        assert torch.equal(gb2, gb) and torch.equal(gb3, gb)


@pytest.mark.parametrize("grad", ["dw", "db"])
def test_layernorm_one_gradient(grad):
    import normalization_row_wise_amd as rn
    wl = workloads.small("layernorm", 2048, 4096, "bf16", seed=220)
    _say("one gradient", grad, wl.name)
    t = workloads.generate(wl)
    d = gp.to_device(t)
    ws = rn.new_workspace(rn.workspace_bytes(wl.M, wl.N, 1), gp.dev())
    dx, gw, gb = _bwd(rn, wl, d, ws, dw=grad == "dw", db=grad == "db")
    torch.cuda.synchronize()
    o = gp.run_oracle(wl, t)
    got = gw if grad == "dw" else gb
    assert (gb if grad == "dw" else gw) is None
    assert gp.f32_report(got.cpu(), o[grad]) <= gp.REL_GRAD


def test_one_workspace_across_shapes_and_ops():
    """One workspace, sized for the largest call, serves a sequence of different
    problems on one stream; each result equals the same call on a fresh workspace."""
    import normalization_row_wise_amd as rn
    cases = [CASES[i] for i in (0, 3, 6, 2, 4, 8, 0)]
    _say("shared workspace", [c.name for c in cases])
    need = max(rn.workspace_bytes(c.M, c.N, _ngrads(c)) for c in cases)
    ws = rn.new_workspace(need, gp.dev())
    for wl in cases:
        d = gp.to_device(workloads.generate(wl))
        shared = _bwd(rn, wl, d, ws)
        fresh = _bwd(rn, wl, d, rn.new_workspace(rn.workspace_bytes(wl.M, wl.N, _ngrads(wl)),
                                                  gp.dev()))
        torch.cuda.synchronize()
        for a, b in zip(shared[1:], fresh[1:]):
            if a is not None:
                assert torch.equal(a, b), wl.name


def test_single_row_with_zero_strides_narrow_layernorm():
    """M = 1 with row strides of 0 through the C ABI: a single row's stride is never
    used, so the idle teams of a narrow workgroup must not land on row 0 again (their
    dy would otherwise be added into db once per idle team)."""
    import normalization_row_wise_amd as rn
    wl = workloads.small("layernorm", 1, 64, "bf16", seed=230)
    _say("single row, zero strides", wl.name)
    t = workloads.generate(wl)
    d = gp.to_device(t)
    N = wl.N
    dx = torch.empty_like(d["dy"])
    gw = torch.full((N,), 3.0, device=gp.dev())
    gb = torch.full((N,), 3.0, device=gp.dev())
    ws = rn.new_workspace(rn.workspace_bytes(1, N, 2), gp.dev())
    vp = lambda a: ctypes.c_void_p(a.data_ptr())
    st = rn.lib.layernorm_bwd(vp(d["dy"]), 0, vp(d["x"]), 0, vp(d["w"]), vp(dx), 0, vp(gw), vp(gb),
                              vp(ws), ws.numel(), 1, N, t["eps"], 2, 2,
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, rn.lib.rn_status_str(st)
    y = torch.empty_like(d["x"])
    res = torch.empty_like(d["x"])
    ro = torch.empty_like(d["x"])
    st = rn.lib.fused_add_rmsnorm_fwd(vp(d["x"]), 0, vp(d["x"]), 0, vp(d["w"]), vp(y), 0, vp(ro),
                                      0, None, 1, N, t["eps"], 0.0, 2, 2,
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    o = gp.run_oracle(wl, t)
    rep = gp.io_report(dx.cpu(), o["dx"], wl.io)
    assert gp.io_ok(rep, wl.io), rep
    assert gp.f32_report(gw.cpu(), o["dw"]) <= gp.REL_GRAD
    assert gp.f32_report(gb.cpu(), o["db"]) <= gp.REL_GRAD
    two_x = (d["x"].float() + d["x"].float()).to(torch.bfloat16)
    assert torch.equal(ro, two_x)
