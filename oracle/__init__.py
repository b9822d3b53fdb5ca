"""Correctness oracle (fp64, CPU, numpy) for the row-wise normalisation path and the
fused linear distillation loss (``oracle.distill``).

TEST INFRASTRUCTURE ONLY.  Imported by the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the product.  It shares no code
with the HIP kernels and never reads their results.

Every function here is pinned by the ``-m "not gpu"`` tests in ``tests/`` against
facts fixed outside this package (worked examples from the pages, closed forms,
invariants, finite differences and torch's own fp64 CPU routines).
"""
from .rounding import DTYPES, from_bits, round_to, to_bits, ulp_distance
from .norms import (
    fused_add_rmsnorm_bwd,
    fused_add_rmsnorm_fwd,
    layernorm_bwd,
    layernorm_fwd,
    rmsnorm_bwd,
    rmsnorm_fwd,
    rmsnorm_fwd_preadd_control,
)

__all__ = [
    "DTYPES", "from_bits", "round_to", "to_bits", "ulp_distance",
    "rmsnorm_fwd", "rmsnorm_bwd", "layernorm_fwd", "layernorm_bwd",
    "fused_add_rmsnorm_fwd", "fused_add_rmsnorm_bwd", "rmsnorm_fwd_preadd_control",
]
