"""GPU parity of the split-row kernels: a few long rows, each spread over several
workgroups that all walk the whole row for its statistics (a decode row, a small
batch).  Compared with the fp64 oracle element by element.  The same calls with the row
kernels forced (a launch-shape override turns the split off) meet the same gates; dx
with frozen parameters is bit-identical to dx with trainable ones; in-place calls, which
must not take the split kernels, stay correct.

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


def _wl(op, m, n, io, wt=None, gemma=False, **kw):
    off = 1.0 if gemma else 0.0
    return workloads.small(op, m, n, io, wt, offset=off, weight="gemma" if gemma else "unit",
                           seed=500 + m + n % 97, **kw)


# Spans are 256 16-byte accesses (2048 elements of a 16-bit type, 1024 of fp32); N not a
# multiple of that leaves a ragged last span.  Rows of many spans at larger row counts
# give each workgroup a run of several spans (the later ones read again after the walk).
CASES = [
    _wl("rmsnorm", 1, 18432, "bf16", "fp32"),           # the decode row
    _wl("rmsnorm", 1, 18432, "fp16"),
    _wl("rmsnorm", 1, 18432, "fp32"),
    _wl("rmsnorm", 1, 4096, "bf16", gemma=True),
    _wl("rmsnorm", 2, 4104, "bf16", gemma=True),         # spans 2048 + 2048 + 8
    _wl("rmsnorm", 128, 4096, "bf16", gemma=True),       # 256 workgroups
    _wl("rmsnorm", 9, 24576, "fp32", "fp32"),            # 24 spans of 1024
    _wl("layernorm", 1, 4096, "bf16"),
    _wl("layernorm", 3, 8200, "bf16"),
    _wl("layernorm", 16, 4104, "fp16", bias=False),
    _wl("layernorm", 5, 24576, "fp32"),
    _wl("layernorm", 2, 18432, "bf16", "fp32"),
    _wl("fused_add_rmsnorm", 1, 18432, "bf16", gemma=True),
    _wl("fused_add_rmsnorm", 4, 8192, "bf16", gemma=True),
    _wl("fused_add_rmsnorm", 7, 12288, "fp16", "fp32", dres=False),
    _wl("fused_add_rmsnorm", 3, 6144, "fp32"),
    _wl("rmsnorm", 128, 18432, "bf16", "fp32"),          # 2 workgroups of 5 / 4 spans
    _wl("rmsnorm", 128, 18432, "fp32"),                  # backward: 2 of 9 spans
    _wl("rmsnorm", 16, 18432, "fp16", gemma=True),
    _wl("layernorm", 100, 8200, "bf16"),                 # 2 of 3 / 2 spans, ragged
    _wl("layernorm", 20, 24576, "fp32", bias=False),     # 12 of 2 spans
    _wl("fused_add_rmsnorm", 60, 12288, "bf16", gemma=True),  # 3 of 2 spans
    _wl("layernorm", 7, 1028, "fp32"),                   # spans of 1024 + 4
    _wl("rmsnorm", 3, 2056, "fp16", "fp32", gemma=True),  # spans of 2048 + 8
    _wl("fused_add_rmsnorm", 128, 4104, "fp16", gemma=True),  # 2 of 2 / 1 spans
    # Rows whose walks would fetch many bytes across XCDs: their workgroups are
    # renumbered onto one XCD per row (grid sizes 161, 117, 110 and 252: not multiples
    # of the 8 XCDs, so some XCDs take one workgroup more than others)
    _wl("rmsnorm", 7, 23552, "fp32"),                    # 23 workgroups of 1 span
    _wl("fused_add_rmsnorm", 13, 18432, "bf16", gemma=True),  # 9 of 1 span
    _wl("fused_add_rmsnorm", 11, 18440, "fp16", "fp32"),  # 10 of 1, ragged last span
    _wl("layernorm", 21, 24568, "bf16"),                  # 12 of 1, ragged last span
]


@pytest.mark.parametrize("wl", CASES, ids=lambda c: c.name)
def test_split_rows_against_oracle(wl):
    _say(wl.name)
    fails = gp.check(wl)
    assert not fails, "\n".join(fails)


@pytest.mark.parametrize("wl", CASES[::3], ids=lambda c: c.name)
def test_row_kernels_on_split_shapes_meet_the_same_gates(wl):
    """The same shapes through the row kernels: outputs that alias their inputs (y == x,
    dx == dy, residual_out == residual) are never split, so these calls run one team
    per row, with the column sum folded into the backward launch."""
    _say("row kernels (in place)", wl.name)
    t = workloads.generate(wl)
    g = gp.run_gpu(wl, t, inplace=True)
    o = gp.run_oracle(wl, t)
    fails = gp.compare(wl, g, o)
    assert not fails, "\n".join(fails)


@pytest.mark.parametrize("wl", CASES[::2], ids=lambda c: c.name)
def test_split_frozen_dx_bit_identical(wl):
    _say("split frozen vs trainable", wl.name)
    t = workloads.generate(wl)
    full = gp.run_gpu(wl, t, dw=True, db=True)
    frozen = gp.run_gpu(wl, t, dw=False, db=False)
    bits = gp._BITS_VIEW[wl.io]
    assert torch.equal(full["dx"].view(bits), frozen["dx"].view(bits))
    again = gp.run_gpu(wl, t, dw=True, db=True)
    assert torch.equal(again["dw"], full["dw"])


@pytest.mark.parametrize("op", ["rmsnorm", "layernorm", "fused_add_rmsnorm"])
def test_inplace_calls_of_split_shapes(op):
    """dx == dy and y == x on a shape that would be split: another workgroup of the row
    would read what this one overwrites, so these calls take the row kernels."""
    import normalization_row_wise_amd as rn
    wl = _wl(op, 2, 8192, "bf16", gemma=op != "layernorm")
    _say("in-place split shape", wl.name)
    t = workloads.generate(wl)
    o = gp.run_oracle(wl, t)
    d = gp.to_device(t)
    if op == "rmsnorm":
        xin = d["x"].clone()
        y, _ = rn.rmsnorm_fwd(xin, d["w"], t["eps"], t["offset"], y=xin)
        dy = d["dy"].clone()
        dx, dw = rn.rmsnorm_bwd(dy, d["x"], d["w"], t["eps"], t["offset"], dx=dy)
    elif op == "layernorm":
        xin = d["x"].clone()
        y, _, _ = rn.layernorm_fwd(xin, d["w"], d["b"], t["eps"], y=xin)
        dy = d["dy"].clone()
        dx, dw, db = rn.layernorm_bwd(dy, d["x"], d["w"], t["eps"], dx=dy)
    else:
        res = d["residual"].clone()
        y, ro, _ = rn.fused_add_rmsnorm_fwd(d["x"], res, d["w"], t["eps"], t["offset"],
                                            residual_out=res)
        dy = d["dy"].clone()
        dx, dw = rn.fused_add_rmsnorm_bwd(dy, ro, d["w"], t["eps"], t["offset"], d["dres"],
                                          dx=dy)
        rep = gp.io_report(ro.cpu(), o["residual_out"], wl.io)
        assert rep["max_ulp"] == 0, rep
    torch.cuda.synchronize()
    assert dx.data_ptr() == dy.data_ptr()
    for k, g in (("y", y), ("dx", dx)):
        rep = gp.io_report(g.cpu(), o[k], wl.io)
        assert gp.io_ok(rep, wl.io), (k, rep)
    assert gp.f32_report(dw.cpu(), o["dw"]) <= gp.REL_GRAD
