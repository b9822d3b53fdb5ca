"""GPU test of rmsnorm_bwd_noalloc, the RMSNorm backward that allocates nothing: its
partial rows of dW live in a per-GPU device array inside the library instead of a
caller's workspace.  Called through the C ABI and compared with rmsnorm_bwd (with a
workspace) bit for bit, on two calls in a row, the second smaller; a call beyond the
array's 8 MiB is refused before anything is enqueued."""
import ctypes

import pytest
import torch

import workloads
from tests import gpu_parity as gp

pytestmark = pytest.mark.gpu

RN_ERR_SCRATCH = -9
DT = {"bf16": 2, "fp16": 1, "fp32": 0}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import __graft_entry__
    __graft_entry__.ensure_built()
    import normalization_row_wise_amd as rn
    return rn


def _noalloc(rn, d, wl, dx, dw):
    vp = lambda a: None if a is None else ctypes.c_void_p(a.data_ptr())
    N = wl.N
    return rn.lib.rmsnorm_bwd_noalloc(
        vp(d["dy"]), N, vp(d["x"]), N, vp(d["w"]), vp(dx), N, vp(dw), wl.M, N, d["eps"],
        d["offset"], DT[wl.io], DT[wl.wt], ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


# the second call is smaller than the first (fewer rows and narrower, so fewer and
# shorter partial rows: whatever the first left in the array must not leak into it)
CALLS = [
    workloads.small("rmsnorm", 8192, 8192, "bf16", seed=301),
    workloads.small("rmsnorm", 777, 3000, "fp16", "fp32", offset=1.0, weight="gemma", seed=302),
]


def test_noalloc_matches_the_workspace_entry_point():
    import normalization_row_wise_amd as rn
    for wl in CALLS:
        print("[case] noalloc", wl.name, flush=True)
        t = workloads.generate(wl)
        d = gp.to_device(t)
        ref_dx, ref_dw = rn.rmsnorm_bwd(d["dy"], d["x"], d["w"], t["eps"], t["offset"])
        dx = torch.full_like(d["dy"], float("nan"))
        dw = torch.full((wl.N,), float("nan"), device=gp.dev())
        st = _noalloc(rn, d, wl, dx, dw)
        assert st == 0, rn.lib.rn_status_str(st)
        torch.cuda.synchronize()
        bits = gp._BITS_VIEW[wl.io]
        assert torch.equal(dx.view(bits), ref_dx.view(bits)), wl.name
        assert torch.equal(dw, ref_dw), wl.name
        o = gp.run_oracle(wl, t)
        rep = gp.io_report(dx.cpu(), o["dx"], wl.io)
        assert gp.io_ok(rep, wl.io), rep
        assert gp.f32_report(dw.cpu(), o["dw"]) <= gp.REL_GRAD


def test_noalloc_frozen_and_binding():
    import normalization_row_wise_amd as rn
    wl = CALLS[1]
    print("[case] noalloc frozen", wl.name, flush=True)
    t = workloads.generate(wl)
    d = gp.to_device(t)
    ref_dx, _ = rn.rmsnorm_bwd(d["dy"], d["x"], d["w"], t["eps"], t["offset"], dw=None)
    dx, dw = rn.rmsnorm_bwd_noalloc(d["dy"], d["x"], d["w"], t["eps"], t["offset"], dw=None)
    dx2, dw2 = rn.rmsnorm_bwd_noalloc(d["dy"], d["x"], d["w"], t["eps"], t["offset"])
    _, ref_dw = rn.rmsnorm_bwd(d["dy"], d["x"], d["w"], t["eps"], t["offset"])
    torch.cuda.synchronize()
    bits = gp._BITS_VIEW[wl.io]
    assert dw is None
    assert torch.equal(dx.view(bits), ref_dx.view(bits))
    assert torch.equal(dx2.view(bits), ref_dx.view(bits)) and torch.equal(dw2, ref_dw)


def test_noalloc_refuses_more_than_its_scratch():
    """4096 rows of 16384: 256 partial rows of 64 KiB = 16 MiB > 8 MiB.  Refused with
    RN_ERR_SCRATCH before any launch: the outputs keep their sentinel values."""
    import normalization_row_wise_amd as rn
    wl = workloads.small("rmsnorm", 4096, 16384, "bf16", seed=303)
    print("[case] noalloc refusal", wl.name, flush=True)
    assert rn.workspace_bytes(wl.M, wl.N, 1) > 8 << 20
    d = {"dy": torch.zeros(wl.M, wl.N, dtype=torch.bfloat16, device=gp.dev()),
         "x": torch.zeros(wl.M, wl.N, dtype=torch.bfloat16, device=gp.dev()),
         "w": torch.ones(wl.N, dtype=torch.bfloat16, device=gp.dev()), "eps": 1e-6, "offset": 0.0}
    dx = torch.full_like(d["dy"], 7.0)
    dw = torch.full((wl.N,), 7.0, device=gp.dev())
    assert _noalloc(rn, d, wl, dx, dw) == RN_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool(torch.all(dx == 7.0)) and bool(torch.all(dw == 7.0))
