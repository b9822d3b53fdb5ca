"""CPU checks of the measurement code in bench.py: the algorithmic byte counts of the
named workloads, and the oracle's CPU-baseline leg."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402

# Minimum bytes per call, each operand once.  Forward: read x (and the residual), write
# y (and residual_out), read w (and b), write the fp32 row statistics (rstd; LayerNorm
# also the mean).  Backward stage 1: read dy and x (the fused add: residual_out and the
# residual-output gradient), write dx, read w; the statistics are recomputed from x,
# so none are read.  Trainable: plus the fp32 dW (and dB) written once.
MiB2 = 2048 * 4096 * 2          # one 2048 x 4096 bf16 tensor
BYTES = {
    # name: (fwd, bwd trainable, bwd frozen)
    "gemma_rmsnorm_128x4096_bf16": (2 * 128 * 4096 * 2 + 4096 * 2 + 128 * 4,
                                    3 * 128 * 4096 * 2 + 4096 * 2 + 4096 * 4,
                                    3 * 128 * 4096 * 2 + 4096 * 2),
    "layernorm_2048x4096_bf16": (2 * MiB2 + 2 * 4096 * 2 + 2048 * 8,
                                 3 * MiB2 + 4096 * 2 + 2 * 4096 * 4,
                                 3 * MiB2 + 4096 * 2),
    "rmsnorm_8192x8192_bf16": (2 * 8192 * 8192 * 2 + 8192 * 2 + 8192 * 4,
                               3 * 8192 * 8192 * 2 + 8192 * 2 + 8192 * 4,
                               3 * 8192 * 8192 * 2 + 8192 * 2),
    "fused_add_rmsnorm_2048x8192_bf16": (4 * 2048 * 8192 * 2 + 8192 * 2 + 2048 * 4,
                                         4 * 2048 * 8192 * 2 + 8192 * 2 + 8192 * 4,
                                         4 * 2048 * 8192 * 2 + 8192 * 2),
    "rmsnorm_1x18432_bf16_w32": (2 * 18432 * 2 + 18432 * 4 + 4,
                                 3 * 18432 * 2 + 18432 * 4 + 18432 * 4,
                                 3 * 18432 * 2 + 18432 * 4),
    "rmsnorm_128x18432_fp32": (2 * 128 * 18432 * 4 + 18432 * 4 + 128 * 4,
                               3 * 128 * 18432 * 4 + 18432 * 4 + 18432 * 4,
                               3 * 128 * 18432 * 4 + 18432 * 4),
}


@pytest.mark.parametrize("name", sorted(BYTES))
def test_algorithmic_bytes(name):
    wl = workloads.BY_NAME[name]
    fwd, bwd_t, bwd_f = BYTES[name]
    t = bench.alg_bytes(wl, True)
    f = bench.alg_bytes(wl, False)
    assert (t["fwd"], t["bwd"], t["step"]) == (fwd, bwd_t, fwd + bwd_t)
    assert (f["fwd"], f["bwd"], f["step"]) == (fwd, bwd_f, fwd + bwd_f)
    assert t["bwd_stage1"] == f["bwd_stage1"] == bwd_f


def test_cpu_baseline_runs_on_the_host():
    import os
    wl = workloads.small("layernorm", 6, 96)
    r = bench.cpu_baseline(wl, 0.05)
    assert r["kind"] == "oracle" and r["value"] > 0
    assert r["cores"] == max(1, min(len(os.sched_getaffinity(0)), bench.CPU_SHARE))
    assert r["single_thread"]["cores"] == 1 and r["single_thread"]["value"] > 0
    assert "6 of 6 rows x 96" in r["sample"]


def test_bench_defaults_to_the_largest_named_workload():
    """The headline line is the largest single-GPU configuration of the named ones."""
    import argparse
    largest = max(workloads.CONFIGS, key=lambda c: c.M * c.N)
    assert largest.name == "rmsnorm_8192x8192_bf16"
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert "default=workloads.RMS_8192x8192.name" in src
    assert workloads.RMS_8192x8192 is largest


def test_median_and_rounds_helpers():
    assert bench.median([3, 1, 2]) == 2
    assert bench.median([4, 1, 3, 2]) == 2.5
    assert bench.PROVIDERS == ("trainable", "frozen", "trainable_aa")
