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

TOL_LOSS = gp.DISTILL_TOL_LOSS    # 2e-4
TOL_DX = gp.DISTILL_TOL_DX        # 4e-3
TOL_DW = gp.DISTILL_TOL_DW        # 3e-3
TOL_DB = gp.DISTILL_TOL_DB        # 1e-4


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


@pytest.mark.parametrize("beta", [0.0, 1.0])
def test_mixture_weight_end_points(beta):
    """beta = 0 or 1: the mixture is the student's (teacher's) distribution itself, so J
    and every gradient vanish (the oracle's closed form); the kernels then take ln M as
    ln S (ln T) and return exact zeros."""
    wl = workloads.DistillWorkload(f"d200_h64_v3000_beta{beta:g}", 200, 64, 64, 3000, 64,
                                   beta=beta, bias=True, seed=11)
    _say(wl.name)
    t = workloads.generate_distill(wl)
    loss, dx, dw, db = _run(wl, t)
    o = _oracle(wl, t)
    assert abs(o["loss"]) < 1e-12 and np.abs(o["dx"]).max() < 1e-12
    assert float(loss[0]) == 0.0
    assert not dx.float().any() and not dw.any() and not db.any()


def test_empty_batch():
    """No tokens: the loss is 0 (the mean over an empty batch is taken as 0, as in the
    oracle) and dW and db are written as zeros over their NaN fill; dx is empty."""
    wl = workloads.DistillWorkload("d0_h64_v300_bias", 0, 64, 64, 300, 16, bias=True, seed=12)
    _say(wl.name)
    t = workloads.generate_distill(wl)
    dw = torch.full((wl.V, wl.H), float("nan"), device=gp.dev())
    db = torch.full((wl.V,), float("nan"), device=gp.dev())
    loss, dx, dw, db = _run(wl, t, dw=dw, db=db)
    o = _oracle(wl, t)
    assert o["loss"] == 0.0 and float(loss[0]) == 0.0
    assert tuple(dx.shape) == (0, wl.H)
    assert not dw.any() and not db.any()


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


@pytest.mark.parametrize("wl", workloads.DISTILL_CONFIGS, ids=lambda c: c.name)
def test_named_size_sampled_tokens(wl):
    """The page's sizes (4096 tokens, H = 4096, V = 128256 and 151936, chunks of 1024):
    dx of 16 sampled tokens against the oracle (each needs only its own logits row), and
    dx and the loss bit-identical for a frozen head."""
    _say(wl.name)
    t = workloads.generate_distill(wl)
    loss, dx, dw, _ = _run(wl, t)
    lf, dxf, dwf, _ = _run(wl, t, dw=None, db=None)
    assert dwf is None and torch.equal(loss, lf)
    assert torch.equal(dx.view(torch.int16), dxf.view(torch.int16))
    assert bool(torch.isfinite(dw).all()) and bool(torch.isfinite(loss).all())
    # adding a constant to a token's student logits leaves the loss unchanged, so each
    # token's logit gradient sums to zero over the vocabulary, and so do the columns of
    # dW (sum over v of dW[v, :] = sum over t of (sum over v of dz[t, v]) xs[t, :]), up to
    # the bf16 rounding of dz (relative 2^-9 per element, summing like a random walk:
    # about 2^-9 / sqrt(V), 5e-6 here, against the column absolute sums)
    col = dw.double().sum(0)
    scale = dw.double().abs().sum(0)
    ratio = float(col.norm() / scale.norm())
    _say(f"dW column sums / column absolute sums: {ratio:.2e}")
    assert ratio <= 1e-4
    rows = np.sort(np.random.default_rng(7).choice(wl.BT, 16, replace=False))
    xs, ws = _f64(t["xs"]), _f64(t["ws"])
    zs = xs[rows] @ ws.T
    zt = _f64(t["xt"])[rows] @ _f64(t["wt"]).T
    _, dj = od.jsd_rows(zs, zt, wl.beta, wl.temperature)
    ref = (dj / wl.BT) @ ws
    assert gp.rel_l2(dx[rows].double().numpy(), ref) <= TOL_DX


def _on_device(t):
    return {k: (v.to(gp.dev()) if v is not None else None) for k, v in t.items()}


def _outputs(wl, dev):
    return (torch.empty(wl.BT, wl.H, dtype=torch.bfloat16, device=dev),
            torch.empty(wl.V, wl.H, dtype=torch.float32, device=dev),
            torch.empty(wl.V, dtype=torch.float32, device=dev) if wl.bias else None)


def _workspace(wl, dev):
    from normalization_row_wise_amd import distill
    need = distill.workspace_bytes(wl.BT, wl.H, wl.Ht, wl.V, wl.chunk, True, True, wl.bias)
    return torch.empty(need + 256, dtype=torch.uint8, device=dev)


def _call(wl, d, outs, ws, stream=None):
    from normalization_row_wise_amd import distill
    dx, dw, db = outs
    return distill.fused_linear_jsd(d["xs"], d["ws"], d["xt"], d["wt"], d["bs"], d["bt"], wl.beta,
                                    wl.temperature, wl.chunk, dx=dx, dw=dw,
                                    db=db if db is not None else None, workspace=ws, stream=stream)


def _same(a, b):
    if a is None or b is None:
        return a is None and b is None
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


def test_graph_capture_replays_match_eager():
    """The call only enqueues kernels (no allocation, synchronisation or memset in the
    library): a captured HIP graph, replayed with new values written into its inputs and
    eager work between the replays, gives the eager call's bits every time."""
    import dataclasses
    wl = CASES[0]
    _say("graph", wl.name)
    dev = gp.dev()
    d = _on_device(workloads.generate_distill(wl))
    outs, ws = _outputs(wl, dev), _workspace(wl, dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            _call(wl, d, outs, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        loss_g = _call(wl, d, outs, ws)[0]
    torch.cuda.synchronize()
    outs_e, ws_e = _outputs(wl, dev), _workspace(wl, dev)
    for seed in (11, 12, 13):
        new = workloads.generate_distill(dataclasses.replace(wl, seed=seed))
        for k, v in new.items():
            if v is not None:
                d[k].copy_(v.to(dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [loss_g.clone()] + [o.clone() if o is not None else None for o in outs]
        loss_e = _call(wl, d, outs_e, ws_e)[0]
        torch.cuda.synchronize()
        want = [loss_e] + list(outs_e)
        for name, a, b in zip(("loss", "dx", "dw", "db"), got, want):
            assert _same(a, b), (seed, name)
    o = _oracle(wl, new)
    assert abs(float(got[0][0]) - o["loss"]) <= TOL_LOSS * abs(o["loss"])
    assert gp.rel_l2(got[1].double().cpu().numpy(), o["dx"]) <= TOL_DX


def test_two_streams_at_once():
    """Two calls in flight on two streams, each with its own workspace and outputs, give
    the bits of the same calls made one after the other."""
    a_wl, b_wl = CASES[0], CASES[2]
    _say("two streams", a_wl.name, b_wl.name)
    dev = gp.dev()
    da, db_ = _on_device(workloads.generate_distill(a_wl)), _on_device(workloads.generate_distill(b_wl))
    oa, ob = _outputs(a_wl, dev), _outputs(b_wl, dev)
    wa, wb = _workspace(a_wl, dev), _workspace(b_wl, dev)
    ra = _call(a_wl, da, oa, wa)
    rb = _call(b_wl, db_, ob, wb)
    torch.cuda.synchronize()
    ref_a = [ra[0].clone()] + [o.clone() if o is not None else None for o in oa]
    ref_b = [rb[0].clone()] + [o.clone() if o is not None else None for o in ob]
    for o in list(oa) + list(ob):
        if o is not None:
            o.fill_(float("nan"))
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    keep = []  # every loss tensor stays alive until the streams are done with it
    for _ in range(3):
        keep.append(_call(a_wl, da, oa, wa, stream=sa)[0])
        keep.append(_call(b_wl, db_, ob, wb, stream=sb)[0])
    torch.cuda.synchronize()
    la, lb = keep[-2], keep[-1]
    for name, x, y in zip(("loss", "dx", "dw", "db"), [la] + list(oa), ref_a):
        assert _same(x, y), ("a", name)
    for name, x, y in zip(("loss", "dx", "dw", "db"), [lb] + list(ob), ref_b):
        assert _same(x, y), ("b", name)
