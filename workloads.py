"""Seeded synthetic inputs for the row-wise normalisation path.

Shared by the oracle-side tests, the GPU parity tests, ``bench.py`` and
``__graft_entry__``.  It holds no arithmetic of the method: it only draws random
numbers (torch CPU generator, float32 draws, cast to the storage type with torch's
round-to-nearest-even casts) and names the workloads.

The distributions follow the pages' accuracy reproduction ("fix(cutedsl): fuse Gemma
RMSNorm weight offset in FP32", PyTorch accuracy comparison and minimal reproduction):
standard-normal activations and upstream gradients, and for the Gemma case a weight of
standard-normal values scaled by 0.01 and stored in bf16, used with offset 1.0.  That
page seeds with 42 on its GPU's generator; its tensors cannot be reproduced here, so
every workload uses a CPU generator seeded with 42 (or the seed given), drawing in the
order listed per workload.  The shapes are the ones the pages benchmark: 2048 x 4096
and 8192 x 8192 for the backward tables of "perf(norm): skip dW/dB calculation when
parameters are frozen (#1067)", Benchmark Results; 128 x 4096, 2048 x 8192 and the
18432-wide rows for the forward tables of the Gemma page, Benchmark results.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

TORCH_DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


@dataclass(frozen=True)
class Workload:
    """One synthetic problem: op, shape, storage types, scalars and the weight recipe."""
    name: str
    op: str                 # "rmsnorm" | "layernorm" | "fused_add_rmsnorm"
    M: int
    N: int
    io: str                 # storage type of x, residual, y, dy, dx, residual_out
    wt: str                 # storage type of w (and b)
    eps: float
    offset: float = 0.0
    weight: str = "unit"    # "unit": w = 1 + 0.1*randn ; "gemma": w = 0.01*randn
    bias: bool = False      # LayerNorm only: b = 0.1*randn
    dres: bool = False      # FusedAddRMSNorm only: a gradient reaches residual_out
    seed: int = 42
    note: str = field(default="", compare=False)


# The five benchmark / parity configurations, by what they are.
GEMMA_RMS_128x4096 = Workload(
    "gemma_rmsnorm_128x4096_bf16", "rmsnorm", 128, 4096, "bf16", "bf16", 1e-6, 1.0, "gemma",
    note="Gemma RMSNorm fwd+bwd, dW trainable")
LAYERNORM_2048x4096 = Workload(
    "layernorm_2048x4096_bf16", "layernorm", 2048, 4096, "bf16", "bf16", 1e-5, 0.0, "unit",
    bias=True, note="LayerNorm fwd+bwd, dW/dB trainable vs frozen")
RMS_8192x8192 = Workload(
    "rmsnorm_8192x8192_bf16", "rmsnorm", 8192, 8192, "bf16", "bf16", 1e-6, 0.0, "unit",
    note="RMSNorm fwd+bwd, dW trainable vs frozen")
FUSED_ADD_2048x8192 = Workload(
    "fused_add_rmsnorm_2048x8192_bf16", "fused_add_rmsnorm", 2048, 8192, "bf16", "bf16", 1e-6,
    1.0, "gemma", dres=True, note="FusedAddRMSNorm fwd+bwd, Gemma offset, residual-output grad")
WIDE_1x18432_MIXED = Workload(
    "rmsnorm_1x18432_bf16_w32", "rmsnorm", 1, 18432, "bf16", "fp32", 1e-6, 0.0, "unit",
    note="decode row, bf16 activations with an fp32 weight")
WIDE_128x18432_MIXED = Workload(
    "rmsnorm_128x18432_bf16_w32", "rmsnorm", 128, 18432, "bf16", "fp32", 1e-6, 0.0, "unit")
WIDE_128x18432_FP16 = Workload(
    "rmsnorm_128x18432_fp16", "rmsnorm", 128, 18432, "fp16", "fp16", 1e-6, 0.0, "unit")
WIDE_128x18432_FP32 = Workload(
    "rmsnorm_128x18432_fp32", "rmsnorm", 128, 18432, "fp32", "fp32", 1e-6, 0.0, "unit")

CONFIGS = [
    GEMMA_RMS_128x4096,
    LAYERNORM_2048x4096,
    RMS_8192x8192,
    FUSED_ADD_2048x8192,
    WIDE_1x18432_MIXED,
    WIDE_128x18432_MIXED,
    WIDE_128x18432_FP16,
    WIDE_128x18432_FP32,
]
# Narrow rows (a per-head norm over the head dimension: many rows of 64-256 elements).
# Not among the five configurations; they measure the narrow-row path.
QKNORM_65536x128 = Workload(
    "rmsnorm_65536x128_bf16", "rmsnorm", 65536, 128, "bf16", "bf16", 1e-6, 0.0, "unit",
    note="per-head RMSNorm over a 128-wide head dimension (4096 tokens x 16 heads)")
QKNORM_32768x256 = Workload(
    "rmsnorm_32768x256_bf16", "rmsnorm", 32768, 256, "bf16", "bf16", 1e-6, 0.0, "unit",
    note="per-head RMSNorm over a 256-wide head dimension (4096 tokens x 8 heads)")
NARROW_LN_65536x64 = Workload(
    "layernorm_65536x64_bf16", "layernorm", 65536, 64, "bf16", "bf16", 1e-5, 0.0, "unit",
    bias=True, note="LayerNorm over 64-wide rows")
EXTRAS = [QKNORM_65536x128, QKNORM_32768x256, NARROW_LN_65536x64]

BY_NAME = {c.name: c for c in CONFIGS + EXTRAS}


def generate(wl: Workload, rows: slice | None = None) -> dict:
    """Draw the workload's tensors on the CPU.

    Draw order: x, residual (fused add), w, b (LayerNorm with bias), dy, dres (fused
    add with a residual-output gradient).  Returns CPU tensors in their storage types
    plus the float32 scalars.  ``rows`` keeps only a slice of the [M, N] tensors (the
    full tensors are still drawn, so the values are those of the full workload).
    """
    g = torch.Generator().manual_seed(wl.seed)
    io = TORCH_DTYPES[wl.io]
    wt = TORCH_DTYPES[wl.wt]
    M, N = wl.M, wl.N

    def act():
        return torch.randn(M, N, generator=g, dtype=torch.float32).to(io)

    out = {"x": act()}
    if wl.op == "fused_add_rmsnorm":
        out["residual"] = act()
    if wl.weight == "gemma":
        out["w"] = (torch.randn(N, generator=g, dtype=torch.float32) * 0.01).to(wt)
    else:
        out["w"] = (1.0 + 0.1 * torch.randn(N, generator=g, dtype=torch.float32)).to(wt)
    if wl.op == "layernorm" and wl.bias:
        out["b"] = (0.1 * torch.randn(N, generator=g, dtype=torch.float32)).to(wt)
    out["dy"] = act()
    if wl.op == "fused_add_rmsnorm" and wl.dres:
        out["dres"] = act()
    if rows is not None:
        for k in ("x", "residual", "dy", "dres"):
            if k in out:
                out[k] = out[k][rows].contiguous()
    out["eps"] = float(torch.tensor(wl.eps, dtype=torch.float32).item())
    out["offset"] = float(torch.tensor(wl.offset, dtype=torch.float32).item())
    return out


def small(op: str, M: int, N: int, io: str = "bf16", wt: str | None = None, *,
          eps: float = 1e-6, offset: float = 0.0, weight: str = "unit", bias: bool = True,
          dres: bool = True, seed: int = 0) -> Workload:
    """An ad-hoc workload for parity sweeps (ragged N, several tiles, edge cases)."""
    return Workload(f"{op}_{M}x{N}_{io}_{wt or io}_s{seed}", op, M, N, io, wt or io, eps,
                    offset, weight, bias, dres, seed)


def as_f64(t: torch.Tensor):
    """Exact fp64 numpy copy of a stored tensor (for the oracle)."""
    return t.detach().to("cpu").double().numpy()


# ---- fused linear JSD distillation loss ---------------------------------------------
# "perf(distillation): skip dW/dB calculation when parameters are frozen", Details:
# B*T = 4096 tokens, H = 4096, V = 128256 (and 151936), chunks of 1024 tokens, bf16.  The
# page gives no value distributions: activations are standard normal and head weights
# normal with standard deviation 1/sqrt(H) (logits of order one), biases 0.1 * normal.

@dataclass(frozen=True)
class DistillWorkload:
    """One synthetic distillation problem: sizes, loss parameters and which parts exist."""
    name: str
    BT: int
    H: int
    Ht: int
    V: int
    chunk: int = 1024
    beta: float = 0.5
    temperature: float = 1.0
    bias: bool = False
    seed: int = 42


DISTILL_4096x4096_V128256 = DistillWorkload("distill_jsd_4096x4096_v128256", 4096, 4096, 4096,
                                            128256)
DISTILL_4096x4096_V151936 = DistillWorkload("distill_jsd_4096x4096_v151936", 4096, 4096, 4096,
                                            151936)
DISTILL_CONFIGS = [DISTILL_4096x4096_V128256, DISTILL_4096x4096_V151936]


def generate_distill(wl: DistillWorkload) -> dict:
    """Draw the distillation inputs on the CPU, in the order xs, ws, bs, xt, wt, bt
    (biases only when wl.bias), float32 draws cast to bf16."""
    g = torch.Generator().manual_seed(wl.seed)
    bf = torch.bfloat16

    def n(*shape, scale=1.0):
        return (torch.randn(*shape, generator=g, dtype=torch.float32) * scale).to(bf)

    out = {"xs": n(wl.BT, wl.H), "ws": n(wl.V, wl.H, scale=wl.H ** -0.5)}
    out["bs"] = n(wl.V, scale=0.1) if wl.bias else None
    out["xt"] = n(wl.BT, wl.Ht)
    out["wt"] = n(wl.V, wl.Ht, scale=wl.Ht ** -0.5)
    out["bt"] = n(wl.V, scale=0.1) if wl.bias else None
    return out
