"""Benchmark: row-wise norm forward + backward on one MI355X.

One step = the whole path on one batch: forward (stats, normalise, affine) and
backward (dx, per-workgroup dW/dB partials, column sum).  Default workload: LayerNorm
2048 x 4096 bf16 with trainable weight and bias.  Prints ONE JSON line.

Timing.  Inputs are resident in HBM before the timed region.  S independent buffer
sets (> 2x the 256 MiB MALL in total) rotate through the steps, and step k runs the
forward on set k and the backward on set k + S/2, so every kernel reads data that the
preceding steps have evicted from L2 and MALL: the numbers are HBM numbers.  The K
timed steps are replayed from a HIP graph (captured once; the library's calls never
allocate or synchronise), bracketed by synchronisation; ms_per_step = wall / K.  The
dominant kernel (backward stage 1) is then timed live with HIP events on the launch
stream over an eager pass of the same steps: an event before the backward call and
the library's stage event between its two kernels.

Algorithmic bytes (what the method must move, once each): forward reads x (and
residual), w (and b) and writes y (and residual_out) and the fp32 row statistics;
backward reads dy, x (or residual_out), dres_out, w and writes dx and fp32 dW/dB.
The backward recomputes the statistics from x, so it reads none.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 * 2**20
PROFILES = os.path.join(ROOT, "profiles")


def source_hash() -> str:
    """Hash of the kernel sources: counter summaries are valid only for this hash."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "normalization_row_wise_amd", "csrc")
    for f in sorted(os.listdir(csrc)) + ["../../../include/rownorm.h"]:
        path = os.path.normpath(os.path.join(csrc, f))
        if os.path.isfile(path):
            h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel_key: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE scaled by a copy kernel's readings), or None when
    the summary is missing or was taken from other kernel sources."""
    path = os.path.join(PROFILES, f"pmc_{workload}.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_hash") != source_hash() or kernel_key not in d.get("kernels", {}):
        return None
    k = d["kernels"][kernel_key]
    return int(round((k["fetch_kib"] * d["fetch_scale"] + k["write_kib"] * d["write_scale"]) * 1024))


def alg_bytes(wl: workloads.Workload, trainable: bool) -> dict:
    bx = 2 if wl.io in ("bf16", "fp16") else 4
    bw = 2 if wl.wt in ("bf16", "fp16") else 4
    M, N = wl.M, wl.N
    mn = M * N * bx
    if wl.op == "layernorm":
        fwd = 2 * mn + N * bw * (2 if wl.bias else 1) + M * 8
        bwd1 = 3 * mn + N * bw
        grads = N * 4 * 2 if trainable else 0
    elif wl.op == "rmsnorm":
        fwd = 2 * mn + N * bw + M * 4
        bwd1 = 3 * mn + N * bw
        grads = N * 4 if trainable else 0
    else:
        fwd = 4 * mn + N * bw + M * 4
        bwd1 = (4 if wl.dres else 3) * mn + N * bw
        grads = N * 4 if trainable else 0
    return {"fwd": fwd, "bwd_stage1": bwd1, "bwd": bwd1 + grads, "step": fwd + bwd1 + grads}


class Sets:
    """S resident copies of one workload's inputs and outputs."""

    def __init__(self, wl, S, trainable, rn, torch):
        self.wl, self.S, self.rn, self.torch = wl, S, rn, torch
        base = workloads.generate(wl)
        dev = torch.device("cuda:0")
        self.eps, self.off = base["eps"], base["offset"]
        M, N = wl.M, wl.N
        self.sets = []
        for s in range(S):
            d = {}
            for k in ("x", "residual", "dy", "dres"):
                if k in base:
                    d[k] = base[k].to(dev) if s == 0 else self.sets[0][k].clone()
            d["w"] = base["w"].to(dev)
            if "b" in base:
                d["b"] = base["b"].to(dev)
            d["y"] = torch.empty_like(d["x"])
            d["dx"] = torch.empty_like(d["x"])
            d["rstd"] = torch.empty(M, dtype=torch.float32, device=dev)
            if wl.op == "layernorm":
                d["mean"] = torch.empty(M, dtype=torch.float32, device=dev)
            if wl.op == "fused_add_rmsnorm":
                d["ro"] = torch.empty_like(d["x"])
            ngr = (2 if wl.op == "layernorm" else 1) if trainable else 0
            d["dw"] = torch.empty(N, dtype=torch.float32, device=dev) if trainable else None
            d["db"] = (torch.empty(N, dtype=torch.float32, device=dev)
                       if trainable and wl.op == "layernorm" else None)
            need = rn.workspace_bytes(M, N, ngr) if ngr else 0
            d["ws"] = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
            self.sets.append(d)
        self.bytes_per_set = sum(v.numel() * v.element_size() for v in self.sets[0].values()
                                 if isinstance(v, torch.Tensor))

    def fwd(self, s):
        d, rn, wl = self.sets[s], self.rn, self.wl
        if wl.op == "rmsnorm":
            rn.rmsnorm_fwd(d["x"], d["w"], self.eps, self.off, y=d["y"], rstd=d["rstd"])
        elif wl.op == "layernorm":
            rn.layernorm_fwd(d["x"], d["w"], d.get("b"), self.eps, y=d["y"], mean=d["mean"],
                             rstd=d["rstd"])
        else:
            rn.fused_add_rmsnorm_fwd(d["x"], d["residual"], d["w"], self.eps, self.off, y=d["y"],
                                     residual_out=d["ro"], rstd=d["rstd"])

    def bwd(self, s):
        d, rn, wl = self.sets[s], self.rn, self.wl
        if wl.op == "rmsnorm":
            rn.rmsnorm_bwd(d["dy"], d["x"], d["w"], self.eps, self.off, dx=d["dx"], dw=d["dw"],
                           workspace=d["ws"])
        elif wl.op == "layernorm":
            rn.layernorm_bwd(d["dy"], d["x"], d["w"], self.eps, dx=d["dx"], dw=d["dw"], db=d["db"],
                             workspace=d["ws"])
        else:
            rn.fused_add_rmsnorm_bwd(d["dy"], d["ro"], d["w"], self.eps, self.off, d.get("dres"),
                                     dx=d["dx"], dw=d["dw"], workspace=d["ws"])

    def step(self, k):
        self.fwd(k % self.S)
        self.bwd((k + self.S // 2) % self.S)


MAX_SETS = 256


def n_sets(bytes_per_set: int) -> int:
    """Buffer sets to rotate through: more than three times the MALL in total, so every
    step reads data evicted from L2 and MALL.  Capped at MAX_SETS: a problem too small to
    reach that (a single decode row) is timed with its sets partly cache-resident."""
    s = 2
    while s * bytes_per_set < 3 * MALL_BYTES and s < MAX_SETS:
        s += 2
    return max(s, 4)


def time_steps(sets, K, W, use_graph, torch):
    """Wall-clock seconds for K steps (after W warmup steps)."""
    stream = torch.cuda.current_stream()
    for k in range(W):
        sets.step(k)
    torch.cuda.synchronize()
    if use_graph:
        # one graph holds a whole number of passes over the sets, at least 64 steps
        G = sets.S * max(1, -(-64 // sets.S))
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for k in range(G):
                    sets.step(k)
        torch.cuda.synchronize()
        reps = max(1, K // G)
        g.replay()  # one untimed replay
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        return time.perf_counter() - t0, reps * G
    t0 = time.perf_counter()
    for k in range(K):
        sets.step(k)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, K


def event_times(sets, n, rn, torch):
    """Per-kernel device times (us) from HIP events on the launch stream.

    The forward kernel and the first backward kernel (dx + partial rows) are launched
    through hipExtLaunchKernel with a start/stop event pair, so each pair brackets
    exactly one kernel (the dispatch records both).  The whole backward call (both
    kernels) is bracketed by ordinary events.  A spin kernel holds the GPU while the
    host enqueues every step, so the GPU then runs them back to back."""
    st = torch.cuda.current_stream()
    mk = lambda: torch.cuda.Event(enable_timing=True)
    ev = [[mk() for _ in range(6)] for _ in range(n)]
    for e in (x for row in ev for x in row):
        e.record(st)                      # materialise the event handles
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2.4e9 * (0.002 + 40e-6 * n)))   # ~ 2 ms + 40 us per step
    for k in range(n):
        f0, f1, b0, b1, c0, c1 = ev[k]
        rn.set_timing_events(0, f0, f1)
        sets.fwd(k % sets.S)
        rn.set_timing_events(0, None, None)
        rn.set_timing_events(1, b0, b1)
        c0.record(st)
        sets.bwd((k + sets.S // 2) % sets.S)
        c1.record(st)
        rn.set_timing_events(1, None, None)
    torch.cuda.synchronize()
    f = [ev[k][0].elapsed_time(ev[k][1]) * 1e3 for k in range(n)]
    b1 = [ev[k][2].elapsed_time(ev[k][3]) * 1e3 for k in range(n)]
    b = [ev[k][4].elapsed_time(ev[k][5]) * 1e3 for k in range(n)]
    med = lambda a: sorted(a)[len(a) // 2]
    mean = lambda a: sum(a) / len(a)
    return {"fwd_us_median": med(f), "bwd_stage1_us_median": med(b1), "bwd_us_median": med(b),
            "bwd_stage1_us_mean": mean(b1), "fwd_us_mean": mean(f)}


def stream_ceiling(sets, n, torch) -> dict:
    """Context for the stage-1 roofline: torch's own elementwise kernel moving the same
    row tensors as the backward's first kernel (2 reads + 1 write; the fused add's 3 + 1),
    on the same rotating buffer sets, timed like the library's kernels (events around
    each launch, queued behind a spin kernel).  No reduction, no fp64: what streaming
    alone reaches on this GPU for this size."""
    fused = sets.wl.op == "fused_add_rmsnorm"
    st = torch.cuda.current_stream()
    mk = lambda: torch.cuda.Event(enable_timing=True)
    ev = [[mk(), mk()] for _ in range(n)]
    for e in (x for row in ev for x in row):
        e.record(st)

    def op(k):
        d = sets.sets[(k + sets.S // 2) % sets.S]
        if fused:
            torch.addcmul(d["dres"], d["dy"], d["ro"], out=d["dx"])
        else:
            torch.mul(d["dy"], d["x"], out=d["dx"])

    for k in range(3):
        op(k)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2.4e9 * (0.002 + 20e-6 * n)))
    for k in range(n):
        ev[k][0].record(st)
        op(k)
        ev[k][1].record(st)
    torch.cuda.synchronize()
    t = sorted(ev[k][0].elapsed_time(ev[k][1]) * 1e3 for k in range(n))[n // 2]
    x = sets.sets[0]["x"]
    nbytes = x.numel() * x.element_size() * (4 if fused else 3)
    return {"op": "torch.addcmul, 3 reads + 1 write" if fused else "torch.mul, 2 reads + 1 write",
            "us_median": round(t, 3), "gbs": round(nbytes / (t * 1e-6) / 1e9, 1)}


def cpu_baseline(wl, budget_s: float) -> dict:
    """The oracle (numpy fp64, as it stands) on a bounded sample of the workload's rows,
    forward + backward: first on one thread, repeated until `budget_s` has passed, then
    on every host core the process may use (at most 16): one thread per core, each
    running the same oracle calls on the sample, in rounds until `budget_s` has passed
    again.  numpy releases the interpreter lock inside its array loops, so the threads
    run in parallel.  Each figure is the median over the repetitions (rounds)."""
    from concurrent.futures import ThreadPoolExecutor
    import numpy as np
    import oracle
    rows = min(wl.M, 256)
    t = workloads.generate(wl, rows=slice(0, rows))
    f = workloads.as_f64
    x, dy, w = f(t["x"]), f(t["dy"]), f(t["w"])
    eps, off = t["eps"], t["offset"]
    b = f(t["b"]) if "b" in t else None
    r = f(t["residual"]) if "residual" in t else None
    dres = f(t["dres"]) if "dres" in t else None
    sub = workloads.Workload(wl.name, wl.op, rows, wl.N, wl.io, wl.wt, wl.eps, wl.offset,
                             wl.weight, wl.bias, wl.dres)
    step_bytes = alg_bytes(sub, True)["step"]

    def step(_=None):
        if wl.op == "rmsnorm":
            oracle.rmsnorm_fwd(x, w, eps, off)
            oracle.rmsnorm_bwd(dy, x, w, eps, off)
        elif wl.op == "layernorm":
            oracle.layernorm_fwd(x, w, b, eps)
            oracle.layernorm_bwd(dy, x, w, eps)
        else:
            _, s_q, _ = oracle.fused_add_rmsnorm_fwd(x, r, w, eps, off, wl.io)
            oracle.fused_add_rmsnorm_bwd(dy, dres, s_q, w, eps, off)

    def timed(run) -> tuple:
        times = []
        t0 = time.perf_counter()
        while len(times) < 3 or time.perf_counter() - t0 < budget_s:
            a = time.perf_counter()
            run()
            times.append(time.perf_counter() - a)
        return float(np.median(times)), len(times), time.perf_counter() - t0

    per, n, el = timed(step)
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    with ThreadPoolExecutor(max_workers=cores) as pool:
        list(pool.map(step, range(cores)))  # start the threads before timing
        per_all, n_all, el_all = timed(lambda: list(pool.map(step, range(cores))))
    return {"value": round(step_bytes / per / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{rows} of {wl.M} rows x {wl.N}, fwd+bwd, median of {n} repetitions "
                      f"in {el:.1f} s (numpy fp64, single thread)",
            "us_per_step_of_sample": round(per * 1e6, 1),
            "all_cores": {"value": round(cores * step_bytes / per_all / 1e9, 4), "unit": "GB/s",
                          "cores": cores,
                          "sample": f"{cores} threads, each the same {rows}-row fwd+bwd; median "
                                    f"of {n_all} rounds in {el_all:.1f} s"},
            "cpu_model": _cpu_model()}


def _cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default=workloads.LAYERNORM_2048x4096.name,
                    choices=sorted(workloads.BY_NAME))
    ap.add_argument("--frozen", action="store_true", help="time the frozen-parameter step")
    ap.add_argument("--eager", action="store_true", help="time eager launches, not a graph")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--event-steps", type=int, default=200)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 3 plain device copies of MIB MiB (counter calibration)")
    args = ap.parse_args()

    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy * 2**20 // 2
        a = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_mib": args.calibrate_copy}), flush=True)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (rows "
              "would shard across GPUs with no communication except one all-reduce of "
              "dW/dB).", file=sys.stderr)
        sys.exit(2)

    import torch
    import __graft_entry__
    __graft_entry__.ensure_built()
    import normalization_row_wise_amd as rn

    wl = workloads.BY_NAME[args.config]
    trainable = not args.frozen
    probe = Sets(wl, 1, trainable, rn, torch)
    S = n_sets(probe.bytes_per_set)
    cold = S * probe.bytes_per_set >= 3 * MALL_BYTES
    del probe
    sets = Sets(wl, S, trainable, rn, torch)

    secs, k = time_steps(sets, args.steps, args.warmup, not args.eager, torch)
    ab = alg_bytes(wl, trainable)
    ms = secs / k * 1e3
    gbs = ab["step"] * k / secs / 1e9
    ev = event_times(sets, args.event_steps, rn, torch)

    # frozen-parameter variant of the same step (context for the pruning)
    other = {}
    if trainable:
        fz = Sets(wl, S, False, rn, torch)
        fsecs, fk = time_steps(fz, args.steps, args.warmup, not args.eager, torch)
        fev = event_times(fz, args.event_steps, rn, torch)
        other = {"frozen_us_per_step": round(fsecs / fk * 1e6, 3),
                 "frozen_bwd_kernel_us": round(fev["bwd_stage1_us_median"], 3)}
        del fz

    ceiling = stream_ceiling(sets, args.event_steps, torch) if "dres" in sets.sets[0] or \
        sets.wl.op != "fused_add_rmsnorm" else None
    stage1_us = ev["bwd_stage1_us_mean"]
    achieved = ab["bwd_stage1"] / (stage1_us * 1e-6) / 1e9
    kernel_key = "bwd_stage1_trainable" if trainable else "bwd_frozen"
    traffic = measured_traffic(wl.name, kernel_key)
    line = {
        "metric": "achieved HBM GB/s (% of peak) & µs/call, bf16 norm fwd+bwd at M×N",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": k,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # arithmetic type: row statistics, LayerNorm outputs and dx are formed in fp64
        # (storage type of the activations: config.io)
        "dtype": "f64",
        "data": "synthetic (seeded CPU randn, no dataset)",
        "config": {"workload": wl.name, "op": wl.op, "M": wl.M, "N": wl.N, "io": wl.io,
                   "weight": wl.wt, "trainable_params": trainable,
                   "timing": "eager" if args.eager else "hip graph replay", "buffer_sets": S,
                   "inputs_cold_in_mall": cold},
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "us_per_call": {"fwd_kernel": round(ev["fwd_us_median"], 3),
                        "bwd_stage1_kernel": round(ev["bwd_stage1_us_median"], 3),
                        "bwd_call_events": round(ev["bwd_us_median"], 3),
                        "step_wall": round(ms * 1e3, 3)},
        **other,
        "roofline": {"kernel": "bwd_kernel (stage 1: dx + dW/dB partial rows)" if trainable
                     else "bwd_kernel (frozen parameters: dx only)",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "alg_bytes_per_launch": ab["bwd_stage1"],
                     "avg_launch_us": round(stage1_us, 3),
                     "stream_ceiling": ceiling},
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
