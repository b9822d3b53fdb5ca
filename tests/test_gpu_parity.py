"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Every case prints what it is before touching the GPU, so a failing run names it.
"""
import numpy as np
import pytest
import torch

import oracle
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


# ---- the named workloads at their full sizes ----------------------------------------

FULL = [c for c in workloads.CONFIGS]


@pytest.mark.parametrize("wl", FULL, ids=lambda c: c.name)
def test_named_workload(wl):
    _say(wl.name)
    fails = gp.check(wl)
    assert not fails, "\n".join(fails)


# Maximum sizes: a million rows of 8 (the narrow path's grid-stride limits) and rows of
# the widest N at thousands of rows; every row compared.
LARGE = [
    workloads.small("rmsnorm", 2**20 + 3, 8, "bf16", offset=1.0, weight="gemma", seed=71),
    workloads.small("layernorm", 3001, 24576, "bf16", seed=72),
    workloads.small("fused_add_rmsnorm", 1500, 24576, "fp32", seed=73),
]


@pytest.mark.parametrize("wl", LARGE, ids=lambda c: c.name)
def test_largest_shapes(wl):
    _say(wl.name)
    fails = gp.check(wl)
    assert not fails, "\n".join(fails)


# ---- ragged shapes, several tiles, every type pair -----------------------------------

RAGGED_N = [1, 7, 64, 100, 511, 512, 513, 1000, 1024, 2050, 4095, 4096, 4097, 8191, 8193,
            12288, 16383, 16385, 18432, 24576]
TYPES = [("bf16", "bf16"), ("fp16", "fp16"), ("fp32", "fp32"), ("bf16", "fp32"), ("fp16", "fp32")]
OPS = ["rmsnorm", "layernorm", "fused_add_rmsnorm"]


def _cases():
    out = []
    for i, n in enumerate(RAGGED_N):
        for j, (io, wt) in enumerate(TYPES):
            op = OPS[(i + j) % 3]
            m = [1, 3, 37, 130][(i + 2 * j) % 4]
            off = 1.0 if op != "layernorm" and (i + j) % 2 else 0.0
            out.append(workloads.small(op, m, n, io, wt, offset=off,
                                       weight="gemma" if off else "unit", seed=100 + 7 * i + j))
    return out


@pytest.mark.parametrize("wl", _cases(), ids=lambda c: c.name)
def test_ragged(wl):
    _say(wl.name)
    fails = gp.check(wl)
    assert not fails, "\n".join(fails)


# ---- frozen parameters ----------------------------------------------------------------

@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("io", ["bf16", "fp32"])
def test_frozen_dx_bit_identical_and_dw_unchanged(op, io):
    import normalization_row_wise_amd as rn
    wl = workloads.small(op, 300, 4096, io, offset=1.0 if op != "layernorm" else 0.0, seed=5)
    _say("frozen", wl.name)
    t = workloads.generate(wl)
    full = gp.run_gpu(wl, t, dw=True, db=True)
    frozen = gp.run_gpu(wl, t, dw=False, db=False)
    assert torch.equal(full["dx"].view(torch.int16 if io != "fp32" else torch.int32),
                       frozen["dx"].view(torch.int16 if io != "fp32" else torch.int32))
    assert frozen["dw"] is None
    if op == "layernorm":
        only_w = gp.run_gpu(wl, t, dw=True, db=False)
        only_b = gp.run_gpu(wl, t, dw=False, db=True)
        assert only_w["db"] is None and only_b["dw"] is None
        assert torch.equal(only_w["dw"], full["dw"]) and torch.equal(only_b["db"], full["db"])
        for r in (only_w, only_b):
            assert torch.equal(r["dx"].view(torch.int32 if io == "fp32" else torch.int16),
                               full["dx"].view(torch.int32 if io == "fp32" else torch.int16))
    # dw is reproducible bit for bit
    again = gp.run_gpu(wl, t, dw=True, db=True)
    assert torch.equal(again["dw"], full["dw"])
    del rn


# Shapes whose frozen backward once took its own row layout (a frozen-only V for wide
# rows and for the fused add): the layout now depends on the operation, N and the type
# only, so dx is bit-identical by construction, fp32 outputs included.
@pytest.mark.parametrize("case", [
    ("fused_add_rmsnorm", 2048, 8192, "bf16", "bf16"),
    ("fused_add_rmsnorm", 300, 8192, "fp32", "fp32"),
    ("fused_add_rmsnorm", 200, 2000, "fp16", "fp16"),
    ("rmsnorm", 128, 18432, "fp32", "fp32"),
    ("rmsnorm", 128, 18432, "bf16", "fp32"),
    ("layernorm", 64, 24576, "fp32", "fp32"),
], ids=lambda c: f"{c[0]}_{c[1]}x{c[2]}_{c[3]}_{c[4]}")
def test_frozen_dx_bit_identical_wide_and_fused(case):
    op, m, n, io, wt = case
    wl = workloads.small(op, m, n, io, wt, offset=1.0 if op != "layernorm" else 0.0,
                         weight="gemma" if op != "layernorm" else "unit", seed=11)
    _say("frozen layout", wl.name)
    t = workloads.generate(wl)
    full = gp.run_gpu(wl, t, dw=True, db=True)
    frozen = gp.run_gpu(wl, t, dw=False, db=False)
    bits = torch.int32 if io == "fp32" else torch.int16
    assert torch.equal(full["dx"].view(bits), frozen["dx"].view(bits))


# Wide 16-bit rows whose trainable backward also loads one row ahead: RMSNorm and
# LayerNorm at 48 elements per lane with a 16-bit weight (exact fp32 products, or with
# a Gemma offset the weight kept packed), and the fused add at 32 elements per lane (at
# 48 it keeps a Gemma weight packed but loads one row at a time).  Rows past 128 take
# the row kernels; the row counts give workgroups an odd and an even number of rows.
# LayerNorm at this width also runs with the bias frozen (dW only) and with the weight
# frozen; with both gradients its two LDS blocks fit at stride 384 (teams of at most 384
# threads), wider teams keep dW's in LDS and dB's in registers.
WIDE_PF = [
    workloads.small("rmsnorm", 1001, 18432, "bf16", seed=81),           # V = 48
    workloads.small("rmsnorm", 517, 20480, "fp16", seed=82),            # V = 48
    workloads.small("rmsnorm", 900, 18432, "bf16", offset=1.0, weight="gemma", seed=86),
    workloads.small("rmsnorm", 300, 24576, "fp16", offset=1.0, weight="gemma", seed=87),
    workloads.small("fused_add_rmsnorm", 600, 18432, "bf16", offset=1.0, weight="gemma",
                    seed=88),                                           # V = 48
    workloads.small("fused_add_rmsnorm", 700, 12288, "bf16", offset=1.0, weight="gemma",
                    seed=83),                                           # V = 32
    workloads.small("fused_add_rmsnorm", 1290, 16384, "fp16", "fp32", dres=False, seed=84),
    # LayerNorm with both gradients at V = 48 and teams of 384 threads: both LDS
    # accumulator blocks at stride 384
    workloads.small("layernorm", 700, 18432, "bf16", seed=89),
    workloads.small("layernorm", 300, 17408, "fp32", seed=90),
    workloads.small("layernorm", 521, 18000, "fp16", "fp32", seed=91),
    # ... and with wider teams: dW's block in LDS, dB's accumulators in VGPRs
    workloads.small("layernorm", 257, 20480, "fp16", seed=92),
    workloads.small("layernorm", 300, 24576, "fp32", seed=93),
    workloads.small("layernorm", 200, 22528, "bf16", "fp32", seed=94),
]


@pytest.mark.parametrize("wl", WIDE_PF, ids=lambda c: c.name)
def test_wide_rows_one_row_ahead(wl):
    _say("wide prefetch", wl.name)
    fails = gp.check(wl)
    assert not fails, "\n".join(fails)
    t = workloads.generate(wl)
    full = gp.run_gpu(wl, t, dw=True, db=True)
    frozen = gp.run_gpu(wl, t, dw=False, db=False)
    bits = torch.int32 if wl.io == "fp32" else torch.int16
    assert torch.equal(full["dx"].view(bits), frozen["dx"].view(bits))


# RMSNorm over 2048 rows or more (the fused add over 8192 or more), with teams of 64,
# 128 or 256 threads that cover at least 2048 elements: the trainable backward runs
# 256-thread workgroups of 4, 2 or 1 teams.  Row counts leave the last workgroups short; N is ragged where the team allows.
RMS_TALL = [
    workloads.small("rmsnorm", 2100, 1500, "bf16", seed=101),    # teams of 64 (V = 32)
    workloads.small("rmsnorm", 2051, 4096, "bf16", seed=102),    # teams of 128
    workloads.small("rmsnorm", 2049, 2048, "fp32", seed=103),    # teams of 128 (V = 16)
    workloads.small("rmsnorm", 2300, 7000, "fp16", offset=1.0, weight="gemma", seed=104),
    # the fused add from 8192 rows on: teams of 256 (one per workgroup; 33 or 32 rows per
    # team, so the three-row prefetch ring ends at different points) and of 128 (two)
    workloads.small("fused_add_rmsnorm", 8193, 4096, "bf16", offset=1.0, weight="gemma",
                    seed=105),
    workloads.small("fused_add_rmsnorm", 8200, 2000, "fp16", seed=106),
    # RMSNorm from 8192 rows with rows up to 8192 wide: one 256-thread team per workgroup
    # (N ragged against the team; 33 or 32 rows per workgroup)
    workloads.small("rmsnorm", 8193, 7176, "bf16", seed=107),
    workloads.small("rmsnorm", 8200, 8000, "fp16", seed=108),
]


@pytest.mark.parametrize("wl", RMS_TALL, ids=lambda c: c.name)
def test_tall_rows_small_workgroups(wl):
    _say("tall rows", wl.name)
    fails = gp.check(wl)
    assert not fails, "\n".join(fails)
    t = workloads.generate(wl)
    full = gp.run_gpu(wl, t, dw=True, db=True)
    frozen = gp.run_gpu(wl, t, dw=False, db=False)
    bits = torch.int32 if wl.io == "fp32" else torch.int16
    assert torch.equal(full["dx"].view(bits), frozen["dx"].view(bits))


@pytest.mark.parametrize("grad", ["dw", "db"])
def test_wide_layernorm_one_gradient(grad):
    wl = workloads.small("layernorm", 300, 18432, "bf16", seed=85)
    _say("wide layernorm", grad, wl.name)
    t = workloads.generate(wl)
    g = gp.run_gpu(wl, t, dw=grad == "dw", db=grad == "db")
    o = gp.run_oracle(wl, t)
    rep = gp.io_report(g["dx"].cpu(), o["dx"], wl.io)
    assert gp.io_ok(rep, wl.io), rep
    assert gp.f32_report(g[grad].cpu(), o[grad]) <= gp.REL_GRAD
    other = "db" if grad == "dw" else "dw"
    assert g[other] is None
    frozen = gp.run_gpu(wl, t, dw=False, db=False)
    assert torch.equal(g["dx"].view(torch.int16), frozen["dx"].view(torch.int16))

# The fused add's trainable backward walks its rows through a ring of three register
# sets (two rows loaded ahead of the one reduced).  Row counts that give each team 3, 4
# and 5 rows end the walk at each point of the ring; every row is checked, and dx must
# still equal the frozen kernel's bit for bit.
@pytest.mark.parametrize("case", [
    (1531, 4096, "bf16", "bf16", True, True),     # two teams per workgroup, 3 rows each
    (2043, 4096, "fp16", "fp32", False, True),    # 4 rows each
    (2555, 4096, "bf16", "fp32", True, True),     # 5 rows each
    (1279, 8192, "bf16", "bf16", True, False),    # one team per workgroup, 5 rows; no dres
    (4000, 2048, "fp16", "fp16", False, True),    # four teams per workgroup, 4 rows each
], ids=lambda c: f"{c[0]}x{c[1]}_{c[2]}_{c[3]}")
def test_fused_add_row_ring(case):
    m, n, io, wt, gemma, dres = case
    wl = workloads.small("fused_add_rmsnorm", m, n, io, wt, offset=1.0 if gemma else 0.0,
                         weight="gemma" if gemma else "unit", dres=dres, seed=13 + m)
    _say("row ring", wl.name)
    fails = gp.check(wl)
    assert not fails, "\n".join(fails)
    t = workloads.generate(wl)
    full = gp.run_gpu(wl, t, dw=True, db=True)
    frozen = gp.run_gpu(wl, t, dw=False, db=False)
    bits = torch.int32 if io == "fp32" else torch.int16
    assert torch.equal(full["dx"].view(bits), frozen["dx"].view(bits))


@pytest.mark.parametrize("op", ["rmsnorm", "fused_add_rmsnorm"])
def test_dw_independent_of_offset(op):
    # the offset is a constant of the weight: dw must not move with it
    import normalization_row_wise_amd as rn
    _say("offset-independence", op)
    wl1 = workloads.small(op, 128, 4096, "bf16", offset=1.0, weight="gemma", seed=9)
    wl0 = workloads.small(op, 128, 4096, "bf16", offset=0.0, weight="gemma", seed=9)
    g1 = gp.run_gpu(wl1, workloads.generate(wl1))
    g0 = gp.run_gpu(wl0, workloads.generate(wl0))
    assert torch.equal(g1["dw"], g0["dw"])
    assert not torch.equal(g1["dx"], g0["dx"])
    del rn


# ---- layouts: strided rows, in-place backward, empty batch ------------------------------

@pytest.mark.parametrize("io", ["bf16", "fp16", "fp32"])
def test_strided_rows_and_inplace_backward(io):
    import normalization_row_wise_amd as rn
    _say("strided+inplace", io)
    M, N, pad = 67, 1000, 24
    wl = workloads.small("rmsnorm", M, N, io, offset=1.0, weight="gemma", seed=11)
    t = workloads.generate(wl)
    o = gp.run_oracle(wl, t)
    td = workloads.TORCH_DTYPES[io]
    big = torch.zeros(M, N + pad, dtype=td, device=gp.dev())
    x = big[:, 3:3 + N]
    x.copy_(t["x"].to(gp.dev()))
    gbig = torch.zeros(M, N + 2 * pad, dtype=td, device=gp.dev())
    dy = gbig[:, 5:5 + N]
    dy.copy_(t["dy"].to(gp.dev()))
    w = t["w"].to(gp.dev())
    ybig = torch.full((M, N + pad), 7.0, dtype=td, device=gp.dev())
    y, _ = rn.rmsnorm_fwd(x, w, t["eps"], t["offset"], y=ybig[:, 1:1 + N])
    dx, dw = rn.rmsnorm_bwd(dy, x, w, t["eps"], t["offset"], dx=dy)   # in place over dy
    torch.cuda.synchronize()
    assert dx.data_ptr() == dy.data_ptr()
    for k, g in (("y", y), ("dx", dx)):
        rep = gp.io_report(g.cpu(), o[k], io)
        assert gp.io_ok(rep, io), (k, rep)
    assert gp.f32_report(dw.cpu(), o["dw"]) <= gp.REL_GRAD
    # padding untouched
    assert torch.all(ybig[:, 0] == 7.0) and torch.all(ybig[:, 1 + N:] == 7.0)


def test_fused_add_inplace_residual_and_layernorm_without_bias():
    import normalization_row_wise_amd as rn
    _say("fused-add in place / layernorm no bias")
    wl = workloads.small("fused_add_rmsnorm", 40, 2048, "bf16", offset=1.0, weight="gemma", seed=12)
    t = workloads.generate(wl)
    o = gp.run_oracle(wl, t)
    d = gp.to_device(t)
    res = d["residual"].clone()
    y, ro, _ = rn.fused_add_rmsnorm_fwd(d["x"], res, d["w"], t["eps"], t["offset"], residual_out=res)
    dres = d["dres"].clone()
    dx, _ = rn.fused_add_rmsnorm_bwd(d["dy"], ro, d["w"], t["eps"], t["offset"], dres, dx=dres,
                                     dw=None)
    torch.cuda.synchronize()
    assert ro.data_ptr() == res.data_ptr()
    for k, g in (("y", y), ("residual_out", ro), ("dx", dx)):
        rep = gp.io_report(g.cpu(), o[k], "bf16")
        assert gp.io_ok(rep, "bf16"), (k, rep)
    wl = workloads.small("layernorm", 33, 3000, "bf16", bias=False, seed=13)
    fails = gp.check(wl)
    assert not fails, fails


def test_empty_batch_gives_zero_parameter_gradients():
    import normalization_row_wise_amd as rn
    _say("M = 0")
    x = torch.empty(0, 512, dtype=torch.bfloat16, device=gp.dev())
    w = torch.ones(512, dtype=torch.bfloat16, device=gp.dev())
    dw = torch.full((512,), 3.0, device=gp.dev())
    db = torch.full((512,), 3.0, device=gp.dev())
    rn.layernorm_bwd(x, x, w, 1e-5, dx=x, dw=dw, db=db)
    y, _ = rn.rmsnorm_fwd(x, w)
    torch.cuda.synchronize()
    assert torch.all(dw == 0) and torch.all(db == 0) and y.shape == (0, 512)


# ---- rounding of the packed converts: ties go to even -----------------------------------

@pytest.mark.parametrize("io", ["bf16", "fp16"])
def test_residual_rounding_ties_to_even(io):
    import normalization_row_wise_amd as rn
    _say("ties", io)
    td = workloads.TORCH_DTYPES[io]
    p = 8 if io == "bf16" else 11
    M, N = 4, 4096
    rng = np.random.default_rng(21)
    # x = k * 2^e (p significant bits), r = 2^(e-p): x + r is halfway between two values
    mant = rng.integers(2**(p - 1), 2**p, size=(M, N)).astype(np.float64)
    e = rng.integers(-4, 4, size=(M, N)).astype(np.float64)
    x64 = mant * 2.0 ** (e - (p - 1)) * np.where(rng.random((M, N)) < 0.5, -1, 1)
    r64 = np.sign(x64) * 2.0 ** (e - p)
    r64[:, ::3] = -r64[:, ::3]
    x = torch.tensor(x64, dtype=torch.float32).to(td)
    r = torch.tensor(r64, dtype=torch.float32).to(td)
    assert np.array_equal(x.double().numpy(), x64) and np.array_equal(r.double().numpy(), r64)
    w = torch.ones(N, dtype=td)
    _, ro, _ = rn.fused_add_rmsnorm_fwd(x.to(gp.dev()), r.to(gp.dev()), w.to(gp.dev()), 1e-6, 0.0)
    torch.cuda.synchronize()
    ref = oracle.round_to(x64 + r64, io)
    assert np.array_equal(gp.gpu_bits(ro.cpu(), io), oracle.to_bits(ref, io))


def test_gemma_worked_example_on_gpu():
    import normalization_row_wise_amd as rn
    from tests.golden import load
    g = load("gemma_rmsnorm_row.txt")
    _say("gemma worked example")
    n = int(g["n"])
    x = torch.zeros(1, n, dtype=torch.bfloat16, device=gp.dev())
    x[0, 0] = g["x0"]
    w = torch.full((n,), g["w"], dtype=torch.bfloat16, device=gp.dev())
    y, _ = rn.rmsnorm_fwd(x, w, g["eps"], g["offset"])
    x32 = torch.ones(1, 1, device=gp.dev())
    y32, _ = rn.rmsnorm_fwd(x32, torch.full((1,), g["w"], device=gp.dev()), 0.0, g["offset"])
    torch.cuda.synchronize()
    assert y[0, 0].item() == g["y0_bf16"]
    assert y32[0, 0].item() == g["fp32_y_n1"]


def test_errors_do_not_launch_on_device():
    import normalization_row_wise_amd as rn
    _say("error statuses")
    x = torch.zeros(4, 64, dtype=torch.bfloat16, device=gp.dev())
    w = torch.ones(64, dtype=torch.float16, device=gp.dev())
    with pytest.raises(rn.RowNormError):
        rn.rmsnorm_fwd(x, w)            # bf16 activations with an fp16 weight
    ws = torch.empty(8, dtype=torch.uint8, device=gp.dev())
    with pytest.raises(rn.RowNormError):
        rn.rmsnorm_bwd(x, x, w.to(torch.bfloat16), workspace=ws)


# ---- one workgroup covering every row: the gradient is written without a column sum ----

@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("m", [1, 3])
def test_single_workgroup_gradient_direct_and_via_workspace(op, m):
    import normalization_row_wise_amd as rn
    _say("direct gradient", op, m)
    wl = workloads.small(op, m, 18432 if op == "rmsnorm" else 4096, "bf16",
                         offset=1.0 if op != "layernorm" else 0.0,
                         weight="gemma" if op != "layernorm" else "unit", seed=60 + m)
    t = workloads.generate(wl)
    d = gp.to_device(t)
    N = wl.N
    aligned = {"dw": torch.full((N,), 7.0, device=gp.dev())}
    buf = torch.full((2 * N + 8,), 7.0, device=gp.dev())
    shifted = {"dw": buf[1:1 + N]}                  # 4-byte aligned only: workspace path
    if op == "layernorm":
        aligned["db"] = torch.full((N,), 7.0, device=gp.dev())
        shifted["db"] = buf[N + 5:2 * N + 5]
    outs = []
    for o in (aligned, shifted):
        if op == "rmsnorm":
            rn.rmsnorm_bwd(d["dy"], d["x"], d["w"], t["eps"], t["offset"], dw=o["dw"])
        elif op == "layernorm":
            rn.layernorm_bwd(d["dy"], d["x"], d["w"], t["eps"], dw=o["dw"], db=o["db"])
        else:
            _, ro, _ = rn.fused_add_rmsnorm_fwd(d["x"], d["residual"], d["w"], t["eps"],
                                                t["offset"])
            rn.fused_add_rmsnorm_bwd(d["dy"], ro, d["w"], t["eps"], t["offset"], d["dres"],
                                     dw=o["dw"])
        outs.append(o)
    torch.cuda.synchronize()
    ref = gp.run_oracle(wl, t)
    for k in outs[0]:
        a, b = outs[0][k] + 0.0, outs[1][k] + 0.0      # +0.0 folds a signed zero
        assert torch.equal(a, b), k
        assert gp.f32_report(a.cpu(), ref[k]) <= gp.REL_GRAD, k
    assert torch.all(buf[0] == 7.0) and torch.all(buf[1 + N:N + 5] == 7.0)


# ---- the accuracy comparison of the Gemma page, on the GPU path -------------------------

def test_gemma_fused_offset_accuracy_against_preadd_control():
    # "fix(cutedsl): fuse Gemma RMSNorm weight offset in FP32", PyTorch accuracy
    # comparison: pre-adding the offset to the bf16 weight costs ~3e-3 relative L2 in y;
    # adding it in fp32 inside the kernel brings y to the bf16 rounding floor.
    import normalization_row_wise_amd as rn
    from tests.golden import load
    g = load("accuracy_magnitudes.txt")
    wl = workloads.GEMMA_RMS_128x4096
    _say("gemma accuracy", wl.name)
    t = workloads.generate(wl)
    d = gp.to_device(t)
    fused, _ = rn.rmsnorm_fwd(d["x"], d["w"], t["eps"], t["offset"])
    w_pre = (t["w"].double() + t["offset"]).to(torch.bfloat16).to(gp.dev())   # bf16(w + 1)
    preadd, _ = rn.rmsnorm_fwd(d["x"], w_pre, t["eps"], 0.0)
    torch.cuda.synchronize()
    ref, _ = oracle.rmsnorm_fwd(workloads.as_f64(t["x"]), workloads.as_f64(t["w"]), t["eps"],
                                t["offset"])
    r16 = oracle.round_to(ref, "bf16")
    e_fused = gp.rel_l2(oracle.from_bits(gp.gpu_bits(fused.cpu(), "bf16"), "bf16"), r16)
    e_pre = gp.rel_l2(oracle.from_bits(gp.gpu_bits(preadd.cpu(), "bf16"), "bf16"), r16)
    assert e_fused <= 1e-4, e_fused
    assert g["rmsnorm_y_before"] / 3 <= e_pre <= g["rmsnorm_y_before"] * 3, e_pre
    assert e_pre > 30 * e_fused
