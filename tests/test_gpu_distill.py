"""GPU parity of the fused linear JSD distillation loss against the fp64 oracle
(oracle/distill.py), through the C ABI of include/distill.h.

Gates (derived from the arithmetic the header states):
  * loss: the logits are exact bf16 products summed in fp32 and the softmax and
    divergence run in fp32 with fp64 row sums: relative error <= 2e-4.
  * dx, dw: the logit gradient is rounded to bf16 (relative error uniform within
    +-2^-9, standard deviation 2^-9/sqrt(3) = 1.1e-3) before the two gradient products;
    dx is stored in bf16 (another 1.1e-3): relative L2 <= 4e-3 for dx, 3e-3 for dw.
  * db: a fixed-order fp32 sum of the fp32 logit gradient: relative L2 <= 1e-4.
  * frozen head ([distill], Details: loss and input gradients unchanged): the loss and
    dx are bit-identical with and without dw / db, and for the forward-only call.
"""
import numpy as np
import pytest
import torch

import oracle.distill as od
import workloads
from tests import gpu_parity as gp

pytestmark = pytest.mark.gpu

TOL_LOSS = 2e-4
TOL_DX = 4e-3
TOL_DW = 3e-3
TOL_DB = 1e-4


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


def _f64(t):
    return None if t is None else t.double().numpy()


def _run(wl, t, **kw):
    from normalization_row_wise_amd import distill
    d = {k: (v.to(gp.dev()) if v is not None else None) for k, v in t.items()}
    out = distill.fused_linear_jsd(d["xs"], d["ws"], d["xt"], d["wt"], d["bs"], d["bt"], wl.beta,
                                   wl.temperature, wl.chunk, **kw)
    torch.cuda.synchronize()
    return [o.cpu() if o is not None else None for o in out]


def _oracle(wl, t):
    return od.fused_linear_jsd(_f64(t["xs"]), _f64(t["ws"]), _f64(t["bs"]), _f64(t["xt"]),
                               _f64(t["wt"]), _f64(t["bt"]), wl.beta, wl.temperature)


CASES = [
    # several GEMM tiles in every direction with ragged edges; chunks that leave a short
    # last chunk (not a multiple of 8 tokens); V not a multiple of 8 (K padding)
    workloads.DistillWorkload("d300_h64_v1000_bias", 300, 64, 64, 1000, 128, bias=True, seed=1),
    workloads.DistillWorkload("d257_h128_ht96_v777", 257, 128, 96, 777, 100, beta=0.3,
                              temperature=2.0, seed=2),
    workloads.DistillWorkload("d64_h256_v4096_b25", 64, 256, 256, 4096, 64, beta=0.25,
                              temperature=0.7, bias=True, seed=3),
    workloads.DistillWorkload("d1_h8_v5", 1, 8, 8, 5, 1, seed=4),
    workloads.DistillWorkload("d1000_h512_v2048_one_chunk", 1000, 512, 512, 2048, 1024,
                              bias=True, seed=5),
]


@pytest.mark.parametrize("wl", CASES, ids=lambda c: c.name)
def test_against_oracle(wl):
    _say(wl.name)
    t = workloads.generate_distill(wl)
    loss, dx, dw, db = _run(wl, t)
    o = _oracle(wl, t)
    assert abs(float(loss[0]) - o["loss"]) <= TOL_LOSS * abs(o["loss"]), (float(loss[0]), o["loss"])
    assert gp.rel_l2(dx.double().numpy(), o["dx"]) <= TOL_DX
    assert gp.rel_l2(dw.double().numpy(), o["dw"]) <= TOL_DW
    if wl.bias:
        assert gp.rel_l2(db.double().numpy(), o["db"]) <= TOL_DB
    else:
        assert db is None


@pytest.mark.parametrize("wl", CASES[:3], ids=lambda c: c.name)
def test_frozen_head_changes_nothing_else(wl):
    """[distill], Details: loss and input gradients unchanged when the head is frozen;
    nothing requested: forward only, same loss.  Repeated calls: identical bits."""
    _say("frozen", wl.name)
    t = workloads.generate_distill(wl)
    loss, dx, dw, db = _run(wl, t)
    loss2, dx2, dw2, db2 = _run(wl, t)
    lf, dxf, dwf, dbf = _run(wl, t, dw=None, db=None)
    l0, dx0, dw0, db0 = _run(wl, t, dx=None, dw=None, db=None)
    assert dwf is None and dbf is None and dx0 is None and dw0 is None and db0 is None
    assert torch.equal(loss, lf) and torch.equal(loss, l0) and torch.equal(loss, loss2)
    assert torch.equal(dx.view(torch.int16), dxf.view(torch.int16))
    assert torch.equal(dx.view(torch.int16), dx2.view(torch.int16)) and torch.equal(dw, dw2)
    # the weight gradient alone (input frozen) equals the trainable call's
    _, dxw, dww, _ = _run(wl, t, dx=None, db=None)
    assert dxw is None and torch.equal(dww, dw)


def test_workspace_smaller_for_a_frozen_head():
    from normalization_row_wise_amd import distill
    wl = workloads.DISTILL_4096x4096_V128256
    full = distill.workspace_bytes(wl.BT, wl.H, wl.Ht, wl.V, wl.chunk, True, True, True)
    frozen = distill.workspace_bytes(wl.BT, wl.H, wl.Ht, wl.V, wl.chunk, True, False, False)
    fwd = distill.workspace_bytes(wl.BT, wl.H, wl.Ht, wl.V, wl.chunk, False, False, False)
    # no dW buffers: the transposed logit gradient (V x chunk bf16) and input chunk
    assert full - frozen >= wl.V * wl.chunk * 2 + wl.H * wl.chunk * 2
    assert fwd < frozen < full


def test_full_vocabulary_mid_batch():
    """V = 128256 (the page's vocabulary) with 512 tokens of 1024: every output against
    the oracle (about half a TFLOP of fp64 products on the host)."""
    wl = workloads.DistillWorkload("d512_h1024_v128256", 512, 1024, 1024, 128256, 256, seed=6)
    _say(wl.name)
    t = workloads.generate_distill(wl)
    loss, dx, dw, _ = _run(wl, t)
    o = _oracle(wl, t)
    assert abs(float(loss[0]) - o["loss"]) <= TOL_LOSS * abs(o["loss"])
    assert gp.rel_l2(dx.double().numpy(), o["dx"]) <= TOL_DX
    assert gp.rel_l2(dw.double().numpy(), o["dw"]) <= TOL_DW


def test_named_size_sampled_tokens():
    """The page's size (4096 tokens, H = 4096, V = 128256, chunks of 1024): dx of 16
    sampled tokens against the oracle (each needs only its own logits row), and dx and
    the loss bit-identical for a frozen head."""
    wl = workloads.DISTILL_4096x4096_V128256
    _say(wl.name)
    t = workloads.generate_distill(wl)
    loss, dx, dw, _ = _run(wl, t)
    lf, dxf, dwf, _ = _run(wl, t, dw=None, db=None)
    assert dwf is None and torch.equal(loss, lf)
    assert torch.equal(dx.view(torch.int16), dxf.view(torch.int16))
    assert bool(torch.isfinite(dw).all()) and bool(torch.isfinite(loss).all())
    rows = np.sort(np.random.default_rng(7).choice(wl.BT, 16, replace=False))
    xs, ws = _f64(t["xs"]), _f64(t["ws"])
    zs = xs[rows] @ ws.T
    zt = _f64(t["xt"])[rows] @ _f64(t["wt"]).T
    _, dj = od.jsd_rows(zs, zt, wl.beta, wl.temperature)
    ref = (dj / wl.BT) @ ws
    assert gp.rel_l2(dx[rows].double().numpy(), ref) <= TOL_DX
