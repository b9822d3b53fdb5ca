"""Helpers that run a workload through the HIP library and through the fp64 oracle and
compare them element by element.  Used by the GPU tests and by
``__graft_entry__.smoke()``; nothing here runs on import.

Gates (the tolerances this path is held to):
  * 16-bit outputs (y, dx, residual_out): against the oracle rounded once to the same
    type, relative L2 <= 1e-4 and at most 1 unit in the last place per element.
  * fp32 outputs of fp32 I/O: relative L2 <= 1e-5.
  * dw / db (fp32 accumulations): relative L2 <= 1e-5.
  * rstd / mean (fp32): relative L2 <= 1e-6.
  * residual_out: bit-exact (x + residual of two stored values, rounded once).
  * dx with frozen parameters: bit-identical to dx with trainable parameters.
  * fused linear JSD loss: loss within 2e-4 relative, dx within 4e-3 and dW within 3e-3
    relative L2, dB within 1e-4.
Every row of every output is compared (check() runs the oracle on chunks of rows).
Relative L2 is ||a - o||_2 / max(||o||_2, 1e-30) in fp64 (the metric of the accuracy
reproduction on "fix(cutedsl): fuse Gemma RMSNorm weight offset in FP32").
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads

REL_IO16 = 1e-4
MAX_ULP16 = 1
REL_F32 = 1e-5
REL_GRAD = 1e-5
REL_STAT = 1e-6
# fused linear JSD distillation loss (derivations in tests/test_gpu_distill.py)
DISTILL_TOL_LOSS = 2e-4
DISTILL_TOL_DX = 4e-3
DISTILL_TOL_DW = 3e-3
DISTILL_TOL_DB = 1e-4

_BITS_VIEW = {"bf16": torch.int16, "fp16": torch.int16, "fp32": torch.int32}
_NP_BITS = {"bf16": np.uint16, "fp16": np.uint16, "fp32": np.uint32}


def dev():
    return torch.device("cuda:0")


def rel_l2(a, o) -> float:
    a = np.asarray(a, np.float64).ravel()
    o = np.asarray(o, np.float64).ravel()
    return float(np.linalg.norm(a - o) / max(np.linalg.norm(o), 1e-30))


def gpu_bits(t: torch.Tensor, dt: str) -> np.ndarray:
    return t.detach().contiguous().view(_BITS_VIEW[dt]).cpu().numpy().view(_NP_BITS[dt])


def io_stats(t: torch.Tensor, ref: np.ndarray, dt: str) -> np.ndarray:
    """Additive comparison statistics of a stored GPU tensor of type dt against the
    fp64 oracle value rounded once to dt: [sum (g - r)^2, sum r^2, max ulp distance,
    elements more than 1 ulp away, NaNs] (sums combine over row chunks; max by max)."""
    gb = gpu_bits(t, dt)
    r = oracle.round_to(ref, dt)
    rb = oracle.to_bits(r, dt)
    ulp = oracle.ulp_distance(gb, rb, dt)
    g = oracle.from_bits(gb, dt).astype(np.float64).ravel()
    r = np.asarray(r, np.float64).ravel()
    d = g - r
    return np.array([float(np.dot(d, d)), float(np.dot(r, r)),
                     float(ulp.max()) if ulp.size else 0.0, float((ulp > 1).sum()),
                     float(np.isnan(g).sum())])


def _report(st: np.ndarray) -> dict:
    return {"rel_l2": float(np.sqrt(st[0]) / max(np.sqrt(st[1]), 1e-30)), "max_ulp": int(st[2]),
            "n_ulp_gt1": int(st[3]), "nan": int(st[4])}


def io_report(t: torch.Tensor, ref: np.ndarray, dt: str) -> dict:
    """Compare a stored GPU tensor of type dt with the fp64 oracle value."""
    return _report(io_stats(t, ref, dt))


def io_ok(rep: dict, dt: str) -> bool:
    if rep["nan"]:
        return False
    if dt == "fp32":
        return rep["rel_l2"] <= REL_F32
    return rep["rel_l2"] <= REL_IO16 and rep["max_ulp"] <= MAX_ULP16


def f32_report(t, ref) -> float:
    return rel_l2(t.detach().double().cpu().numpy(), ref)


def to_device(tensors: dict) -> dict:
    out = {}
    for k, v in tensors.items():
        out[k] = v.to(dev()) if isinstance(v, torch.Tensor) else v
    return out


def run_gpu(wl: workloads.Workload, t: dict, *, dw: bool = True, db: bool = True,
            inplace: bool = False) -> dict:
    """Forward then backward on the GPU; returns CPU copies of every output.  inplace:
    y overwrites (a copy of) x, residual_out a copy of the residual, dx a copy of dy."""
    import normalization_row_wise_amd as rn
    d = to_device(t)
    out = {}
    if wl.op == "rmsnorm":
        xin = d["x"].clone() if inplace else d["x"]
        y, rstd = rn.rmsnorm_fwd(xin, d["w"], d["eps"], d["offset"], y=xin if inplace else None)
        dy = d["dy"].clone() if inplace else d["dy"]
        dx, dw_ = rn.rmsnorm_bwd(dy, d["x"], d["w"], d["eps"], d["offset"],
                                 dx=dy if inplace else None, dw=True if dw else None)
        out.update(y=y, rstd=rstd, dx=dx, dw=dw_)
    elif wl.op == "layernorm":
        xin = d["x"].clone() if inplace else d["x"]
        y, mean, rstd = rn.layernorm_fwd(xin, d["w"], d.get("b"), d["eps"],
                                         y=xin if inplace else None)
        dy = d["dy"].clone() if inplace else d["dy"]
        dx, dw_, db_ = rn.layernorm_bwd(dy, d["x"], d["w"], d["eps"], dx=dy if inplace else None,
                                        dw=True if dw else None, db=True if db else None)
        out.update(y=y, mean=mean, rstd=rstd, dx=dx, dw=dw_, db=db_)
    else:
        res = d["residual"].clone() if inplace else d["residual"]
        y, ro, rstd = rn.fused_add_rmsnorm_fwd(d["x"], res, d["w"], d["eps"], d["offset"],
                                               residual_out=res if inplace else None)
        dy = d["dy"].clone() if inplace else d["dy"]
        dx, dw_ = rn.fused_add_rmsnorm_bwd(dy, ro, d["w"], d["eps"], d["offset"],
                                           d.get("dres"), dx=dy if inplace else None,
                                           dw=True if dw else None)
        out.update(y=y, residual_out=ro, rstd=rstd, dx=dx, dw=dw_)
    torch.cuda.synchronize()
    return {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in out.items()}


def run_oracle(wl: workloads.Workload, t: dict, rows=None, keep_grads: bool = False) -> dict:
    """The oracle on the same inputs, optionally only on a subset of rows.  For a subset
    the parameter gradients (sums over every row) are dropped, unless keep_grads: then
    they are the subset's own column sums (chunks of rows add up to the whole)."""
    f = workloads.as_f64
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    x, dy, w = sel(f(t["x"])), sel(f(t["dy"])), f(t["w"])
    eps, off = t["eps"], t["offset"]
    out = {}
    if wl.op == "rmsnorm":
        out["y"], out["rstd"] = oracle.rmsnorm_fwd(x, w, eps, off)
        out["dx"], out["dw"] = oracle.rmsnorm_bwd(dy, x, w, eps, off)
    elif wl.op == "layernorm":
        b = f(t["b"]) if "b" in t else None
        out["y"], out["mean"], out["rstd"] = oracle.layernorm_fwd(x, w, b, eps)
        out["dx"], out["dw"], out["db"] = oracle.layernorm_bwd(dy, x, w, eps)
    else:
        r = sel(f(t["residual"]))
        out["y"], out["residual_out"], out["rstd"] = oracle.fused_add_rmsnorm_fwd(
            x, r, w, eps, off, wl.io)
        dres = sel(f(t["dres"])) if "dres" in t else None
        out["dx"], out["dw"] = oracle.fused_add_rmsnorm_bwd(dy, dres, out["residual_out"], w, eps,
                                                            off)
    if rows is not None and not keep_grads:
        out.pop("dw", None)
        out.pop("db", None)
    return out


def compare(wl: workloads.Workload, g: dict, o: dict, rows=None) -> list[str]:
    """Every gate that fails, as readable strings (empty list = parity)."""
    fails = []
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    for k in ("y", "dx", "residual_out"):
        if k in o:
            rep = io_report(sel(g[k]), o[k], wl.io)
            if not io_ok(rep, wl.io):
                fails.append(f"{wl.name} {k}: {rep}")
            if k == "residual_out" and rep["max_ulp"] != 0:
                fails.append(f"{wl.name} residual_out not bit-exact: {rep}")
    for k in ("rstd", "mean"):
        if k in o and g.get(k) is not None:
            e = f32_report(sel(g[k]), o[k])
            if not e <= REL_STAT:
                fails.append(f"{wl.name} {k}: rel_l2 {e:.3e}")
    for k in ("dw", "db"):
        if k in o and g.get(k) is not None:
            e = f32_report(g[k], o[k])
            if not e <= REL_GRAD:
                fails.append(f"{wl.name} {k}: rel_l2 {e:.3e}")
    return fails


# Rows per oracle chunk in check(): about 4 Mi elements (fp64 temporaries of a few
# tens of MB), so that every row of the largest workloads is compared.
CHUNK_ELEMS = 1 << 22


def compare_all_rows(wl: workloads.Workload, g: dict, t: dict) -> list[str]:
    """compare() over every row of the workload, running the oracle on chunks of rows:
    per-element gates on all M rows, relative L2 over the whole tensors, and dw / db
    against the sum of the chunks' column sums (fp64)."""
    M = wl.M
    chunk = max(1, CHUNK_ELEMS // wl.N)
    io, stat, grads = {}, {}, {}
    for r0 in range(0, max(M, 1), chunk):
        rows = slice(r0, min(M, r0 + chunk))
        o = run_oracle(wl, t, rows, keep_grads=True)
        for k in ("y", "dx", "residual_out"):
            if k in o:
                st = io_stats(g[k][rows], o[k], wl.io)
                if k in io:
                    io[k][[0, 1, 3, 4]] += st[[0, 1, 3, 4]]
                    io[k][2] = max(io[k][2], st[2])
                else:
                    io[k] = st
        for k in ("rstd", "mean"):
            if k in o and g.get(k) is not None:
                a = g[k][rows].double().numpy()
                dd = a - o[k]
                stat[k] = stat.get(k, np.zeros(2)) + [float(np.dot(dd, dd)),
                                                      float(np.dot(o[k], o[k]))]
        for k in ("dw", "db"):
            if k in o:
                grads[k] = grads.get(k, 0.0) + o[k]
    fails = []
    for k, st in io.items():
        rep = _report(st)
        if not io_ok(rep, wl.io):
            fails.append(f"{wl.name} {k}: {rep}")
        if k == "residual_out" and rep["max_ulp"] != 0:
            fails.append(f"{wl.name} residual_out not bit-exact: {rep}")
    for k, (sd, sr) in stat.items():
        e = float(np.sqrt(sd) / max(np.sqrt(sr), 1e-30))
        if not e <= REL_STAT:
            fails.append(f"{wl.name} {k}: rel_l2 {e:.3e}")
    for k, ref in grads.items():
        if g.get(k) is not None:
            e = f32_report(g[k], ref)
            if not e <= REL_GRAD:
                fails.append(f"{wl.name} {k}: rel_l2 {e:.3e}")
    return fails


def check(wl: workloads.Workload) -> list[str]:
    """Forward + backward on the GPU against the oracle, every row compared."""
    t = workloads.generate(wl)
    g = run_gpu(wl, t)
    return compare_all_rows(wl, g, t)


def distill_check(wl: workloads.DistillWorkload) -> list[str]:
    """The fused linear JSD loss and its gradients on the GPU against the fp64 oracle."""
    import oracle.distill as od
    from normalization_row_wise_amd import distill
    t = workloads.generate_distill(wl)
    d = {k: (v.to(dev()) if v is not None else None) for k, v in t.items()}
    loss, dx, dw, db = distill.fused_linear_jsd(d["xs"], d["ws"], d["xt"], d["wt"], d["bs"],
                                                d["bt"], wl.beta, wl.temperature, wl.chunk)
    torch.cuda.synchronize()
    f = lambda a: None if a is None else a.double().numpy()  # noqa: E731
    o = od.fused_linear_jsd(f(t["xs"]), f(t["ws"]), f(t["bs"]), f(t["xt"]), f(t["wt"]),
                            f(t["bt"]), wl.beta, wl.temperature)
    fails = []
    got = float(loss[0].cpu())
    if not abs(got - o["loss"]) <= DISTILL_TOL_LOSS * abs(o["loss"]):
        fails.append(f"{wl.name} loss: {got} vs {o['loss']}")
    for k, v, tol in (("dx", dx, DISTILL_TOL_DX), ("dw", dw, DISTILL_TOL_DW),
                      ("db", db, DISTILL_TOL_DB)):
        if v is None:
            continue
        e = rel_l2(v.cpu().double().numpy(), o[k])
        if not e <= tol:
            fails.append(f"{wl.name} {k}: rel_l2 {e:.3e}")
    return fails


def smoke_check() -> None:
    """One small forward + backward of every operation, and one small fused linear JSD
    loss with its gradients, on cuda:0 against the oracle."""
    assert torch.cuda.is_available(), "smoke needs a GPU"
    cases = [
        workloads.small("rmsnorm", 8, 4096, "bf16", eps=1e-6, offset=1.0, weight="gemma", seed=42),
        workloads.small("layernorm", 8, 1000, "bf16", eps=1e-5, seed=1),
        workloads.small("fused_add_rmsnorm", 8, 4096, "bf16", eps=1e-6, offset=1.0,
                        weight="gemma", seed=2),
    ]
    fails = []
    for wl in cases:
        fails += check(wl)
    dl = workloads.DistillWorkload("d96_h64_v1000_bias", 96, 64, 64, 1000, 32, bias=True,
                                   seed=3)
    fails += distill_check(dl)
    assert not fails, "\n".join(fails)
    print("smoke ok:", ", ".join([c.name for c in cases] + [dl.name]), flush=True)
