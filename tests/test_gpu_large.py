"""Row tensors larger than 4 GiB, so that row offsets pass 2^32 bytes.

The inputs are built on the GPU from 63 seeded base rows: row i of x (and of the
residual and its gradient) is base row i mod 63.  The period is odd, so it divides no
power of two: an access that wrapped at 2^32 bytes would land on a row holding other
values.  dy is base row i mod 63 on the active rows (the first 64, 64 on each side of
the 2^32-byte mark, the last 64) and zero elsewhere, so the parameter gradients are sums
over those rows only and the oracle computes them exactly.  Checks:
  * rows 0..62 against the oracle gates;
  * every active row, and a few rows past the mark, bit-identical in y (and
    residual_out) to its twin among rows 0..62, and in dx for the active rows: a row's
    result depends on its values, not on where it lies;
  * dw / db against the oracle over the active rows;
  * dx bit-identical with the parameters frozen.
"""
import numpy as np
import pytest
import torch

import workloads
from tests import gpu_parity as gp

pytestmark = pytest.mark.gpu

BASE = 63

# (op, N, storage type, Gemma offset): rows of N elements, M chosen so that the row
# tensors pass 4 GiB by 4133 rows
CASES = [
    ("rmsnorm", 4096, "bf16", True),
    ("layernorm", 4096, "bf16", False),
    ("fused_add_rmsnorm", 2048, "fp32", True),
    ("rmsnorm", 64, "bf16", False),           # narrow rows: 8-lane teams
]

_BITS = {"bf16": torch.int16, "fp16": torch.int16, "fp32": torch.int32}
_EB = {"bf16": 2, "fp16": 2, "fp32": 4}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import __graft_entry__
    __graft_entry__.ensure_built()


def _run(op, d, w, b, eps, off, trainable):
    import normalization_row_wise_amd as rn
    g = True if trainable else None
    if op == "rmsnorm":
        y, _ = rn.rmsnorm_fwd(d["x"], w, eps, off)
        dx, dw = rn.rmsnorm_bwd(d["dy"], d["x"], w, eps, off, dw=g)
        return dict(y=y, dx=dx, dw=dw)
    if op == "layernorm":
        y, _, _ = rn.layernorm_fwd(d["x"], w, b, eps)
        dx, dw, db = rn.layernorm_bwd(d["dy"], d["x"], w, eps, dw=g, db=g)
        return dict(y=y, dx=dx, dw=dw, db=db)
    y, ro, _ = rn.fused_add_rmsnorm_fwd(d["x"], d["residual"], w, eps, off)
    dx, dw = rn.fused_add_rmsnorm_bwd(d["dy"], ro, w, eps, off, d["dres"], dw=g)
    return dict(y=y, residual_out=ro, dx=dx, dw=dw)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_n{c[1]}_{c[2]}")
def test_rows_past_4gib(case):
    op, N, io, gemma = case
    eb = _EB[io]
    mark = (1 << 32) // (N * eb)             # first row at or past byte 2^32
    M = mark + 4133
    dev = gp.dev()
    wl = workloads.small(op, BASE, N, io, offset=1.0 if gemma else 0.0,
                         weight="gemma" if gemma else "unit", seed=77 + N)
    print("[case] past 4 GiB", op, f"{M}x{N}", io, f"mark row {mark}", flush=True)
    t = workloads.generate(wl)
    active = np.concatenate([np.arange(64), np.arange(mark - 64, mark + 64),
                             np.arange(M - 64, M)])
    idx = torch.arange(M, device=dev) % BASE
    d = {k: t[k].to(dev)[idx] for k in ("x", "residual", "dres") if k in t}
    act = torch.from_numpy(active).to(dev)
    d["dy"] = torch.zeros(M, N, dtype=t["dy"].dtype, device=dev)
    d["dy"][act] = t["dy"].to(dev)[act % BASE]
    w = t["w"].to(dev)
    b = t["b"].to(dev) if "b" in t else None
    g = _run(op, d, w, b, t["eps"], t["offset"], trainable=True)
    frozen_dx = _run(op, d, w, b, t["eps"], t["offset"], trainable=False)["dx"]
    torch.cuda.synchronize()
    bits = _BITS[io]
    assert torch.equal(g["dx"].view(bits), frozen_dx.view(bits))
    del frozen_dx

    # rows 0..62 against the oracle
    head = {k: g[k][:BASE].cpu() for k in ("y", "dx", "residual_out") if k in g}
    o = gp.run_oracle(wl, t)
    for k, v in head.items():
        rep = gp.io_report(v, o[k], io)
        assert gp.io_ok(rep, io), (k, rep)
        if k == "residual_out":
            assert rep["max_ulp"] == 0, rep

    # position independence: twins among rows 0..62
    extra = np.array([mark - 1, mark, mark + 1, mark + 2047, M - 1])
    for k in ("y", "residual_out", "dx"):
        if k not in g:
            continue
        rows = active if k == "dx" else np.unique(np.concatenate([active, extra]))
        r = torch.from_numpy(rows).to(dev)
        got = g[k][r].view(bits)
        want = g[k][r % BASE].view(bits)
        same = (got == want).all(dim=1).cpu().numpy()
        assert same.all(), (k, rows[~same][:8])

    # parameter gradients: sums over the active rows
    ta = dict(t)
    for k in ("x", "residual", "dy", "dres"):
        if k in t:
            ta[k] = t[k][torch.from_numpy(active % BASE)]
    wla = workloads.small(op, len(active), N, io, offset=wl.offset, weight=wl.weight,
                          seed=wl.seed)
    oa = gp.run_oracle(wla, ta)
    for k in ("dw", "db"):
        if g.get(k) is not None:
            e = gp.f32_report(g[k].cpu(), oa[k])
            assert e <= gp.REL_GRAD, (k, e)
