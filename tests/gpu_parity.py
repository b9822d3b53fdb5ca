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


def io_report(t: torch.Tensor, ref: np.ndarray, dt: str) -> dict:
    """Compare a stored GPU tensor of type dt with the fp64 oracle value."""
    gb = gpu_bits(t, dt)
    r = oracle.round_to(ref, dt)
    rb = oracle.to_bits(r, dt)
    ulp = oracle.ulp_distance(gb, rb, dt)
    g = oracle.from_bits(gb, dt)
    return {"rel_l2": rel_l2(g, r), "max_ulp": int(ulp.max()) if ulp.size else 0,
            "n_ulp_gt1": int((ulp > 1).sum()), "nan": int(np.isnan(g).sum())}


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


def run_gpu(wl: workloads.Workload, t: dict, *, dw: bool = True, db: bool = True) -> dict:
    """Forward then backward on the GPU; returns CPU copies of every output."""
    import normalization_row_wise_amd as rn
    d = to_device(t)
    out = {}
    if wl.op == "rmsnorm":
        y, rstd = rn.rmsnorm_fwd(d["x"], d["w"], d["eps"], d["offset"])
        dx, dw_ = rn.rmsnorm_bwd(d["dy"], d["x"], d["w"], d["eps"], d["offset"],
                                 dw=True if dw else None)
        out.update(y=y, rstd=rstd, dx=dx, dw=dw_)
    elif wl.op == "layernorm":
        y, mean, rstd = rn.layernorm_fwd(d["x"], d["w"], d.get("b"), d["eps"])
        dx, dw_, db_ = rn.layernorm_bwd(d["dy"], d["x"], d["w"], d["eps"],
                                        dw=True if dw else None, db=True if db else None)
        out.update(y=y, mean=mean, rstd=rstd, dx=dx, dw=dw_, db=db_)
    else:
        y, ro, rstd = rn.fused_add_rmsnorm_fwd(d["x"], d["residual"], d["w"], d["eps"], d["offset"])
        dx, dw_ = rn.fused_add_rmsnorm_bwd(d["dy"], ro, d["w"], d["eps"], d["offset"],
                                           d.get("dres"), dw=True if dw else None)
        out.update(y=y, residual_out=ro, rstd=rstd, dx=dx, dw=dw_)
    torch.cuda.synchronize()
    return {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in out.items()}


def run_oracle(wl: workloads.Workload, t: dict, rows=None) -> dict:
    """The oracle on the same inputs (optionally only on a subset of rows; then no
    parameter gradients, which need every row)."""
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
    if rows is not None:
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


def check(wl: workloads.Workload, sample_rows: int | None = None) -> list[str]:
    t = workloads.generate(wl)
    g = run_gpu(wl, t)
    rows = None
    if sample_rows is not None and wl.M > sample_rows:
        rows = np.sort(np.random.default_rng(1).choice(wl.M, sample_rows, replace=False))
    o = run_oracle(wl, t, rows)
    fails = compare(wl, g, o, rows)
    if rows is not None:  # parameter gradients need every row
        o_full = run_oracle(wl, t)
        for k in ("dw", "db"):
            if k in o_full and g.get(k) is not None:
                e = f32_report(g[k], o_full[k])
                if not e <= REL_GRAD:
                    fails.append(f"{wl.name} {k}: rel_l2 {e:.3e}")
    return fails


def smoke_check() -> None:
    """One small forward + backward of every operation on cuda:0 against the oracle."""
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
    assert not fails, "\n".join(fails)
    print("smoke ok:", ", ".join(c.name for c in cases), flush=True)
