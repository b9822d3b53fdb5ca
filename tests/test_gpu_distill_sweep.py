"""A seeded sweep of random fused linear JSD problems against the fp64 oracle
(oracle/distill.py), through the C ABI of include/distill.h, with the gates of
tests/test_gpu_distill.py; for each, a frozen head (no dW, no db) leaves the loss and dx
bit-identical ([distill], Details).

Draws: tokens log-uniform over 1..1200, hidden sizes of the two heads multiples of 8 up
to 768 (equal half the time), vocabulary log-uniform over 2..6000, chunks log-uniform
over 1..1024, mixture weight uniform over 0.05..0.95, temperature log-uniform over
0.5..3, biases at random.  Every fourth draw takes a chunk longer than the vocabulary,
so the logits products have more rows than columns.  The oracle's products stay within
about 2e10 multiply-adds per case.
"""
import numpy as np
import pytest
import torch

import workloads
from tests import gpu_parity as gp
from tests.test_gpu_distill import TOL_DB, TOL_DW, TOL_DX, TOL_LOSS, _oracle, _run

pytestmark = pytest.mark.gpu

MAX_MACS = 2e10


def _log_uniform(rng, lo, hi):
    return int(np.clip(round(np.exp(rng.uniform(np.log(lo), np.log(hi)))), lo, hi))


def _draws(n=64, seed=0xD157):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        H = 8 * int(rng.integers(1, 97))
        Ht = H if rng.integers(2) else 8 * int(rng.integers(1, 97))
        chunk = _log_uniform(rng, 1, 1024)
        if i % 4 == 3:
            chunk = max(chunk, 64)
            V = _log_uniform(rng, 2, chunk - 1)
        else:
            V = _log_uniform(rng, 2, 6000)
        BT = _log_uniform(rng, 1, 1200)
        BT = max(1, min(BT, int(MAX_MACS // (V * (H + Ht)))))
        beta = float(rng.uniform(0.05, 0.95))
        tau = float(np.exp(rng.uniform(np.log(0.5), np.log(3.0))))
        bias = bool(rng.integers(2))
        name = f"d{BT}_h{H}_ht{Ht}_v{V}_c{chunk}_b{beta:.2f}_t{tau:.2f}{'_bias' if bias else ''}"
        out.append(workloads.DistillWorkload(name, BT, H, Ht, V, chunk, beta=beta,
                                             temperature=tau, bias=bias, seed=2000 + i))
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
    print("[case] distill sweep", wl.name, flush=True)
    t = workloads.generate_distill(wl)
    loss, dx, dw, db = _run(wl, t)
    o = _oracle(wl, t)
    assert abs(float(loss[0]) - o["loss"]) <= TOL_LOSS * abs(o["loss"]), (float(loss[0]), o["loss"])
    assert gp.rel_l2(dx.double().numpy(), o["dx"]) <= TOL_DX
    assert gp.rel_l2(dw.double().numpy(), o["dw"]) <= TOL_DW
    if wl.bias:
        assert gp.rel_l2(db.double().numpy(), o["db"]) <= TOL_DB
    lf, dxf, dwf, dbf = _run(wl, t, dw=None, db=None)
    assert dwf is None and dbf is None
    assert torch.equal(loss, lf) and torch.equal(dx.view(torch.int16), dxf.view(torch.int16))
