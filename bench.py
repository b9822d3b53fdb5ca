"""Benchmark: row-wise norm forward + backward on one MI355X.

One step = the whole path on one batch: forward (statistics, normalise, affine) and
backward (dx and, for trainable parameters, the per-workgroup dW/dB partial rows, then
the second kernel's fixed-order column sum).
Default workload: RMSNorm 8192 x 8192 bf16 with a trainable weight, the largest of the
named configurations.  Prints ONE JSON line.

Timing protocol (after the Gemma page's "Benchmark results and measurement details":
median of shuffled-provider rounds with an identical A/A duplicate as a control):
  * Inputs are resident in HBM before any timed region.  S independent buffer sets
    (more than three times the 256 MiB MALL in total) rotate through the steps: step k
    runs the forward on set k and the backward on set k + S/2, so every kernel reads
    data the preceding steps have evicted from L2 and MALL.
  * Three providers, each a HIP graph of exactly --steps steps: "trainable", "frozen"
    (dW/dB pruned: null outputs) and "trainable_aa", a second, identical capture of the
    trainable step.  Each round replays every provider once, in a shuffled order, each
    replay bracketed by synchronisation and timed with HIP events on its stream.
  * Reported: the median over --rounds rounds of each provider's time per step; the
    headline value is the trainable provider's; aa_delta_pct compares the two trainable
    captures (run-to-run noise of the protocol itself).
  * Per-kernel times (the roofline): an eager pass of the same steps queued behind a
    spin kernel.  The forward kernel and the backward's first kernel (dx and the
    partial rows) are launched with HIP events that the dispatch itself records (the
    library's instrumentation hook, per thread); the whole backward call is bracketed
    by ordinary HIP events on the launch stream.

Algorithmic bytes (what the method must move, once each): forward reads x (and the
residual), w (and b) and writes y (and residual_out) and the fp32 row statistics;
backward reads dy, x (or residual_out), dres_out, w and writes dx and the fp32 dW/dB.
The backward recomputes the statistics from x, so it reads none.
"""
from __future__ import annotations

import argparse
import json
import os
import random
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
    for f in sorted(f for f in os.listdir(csrc) if f.startswith("rn_")) + [
            "../../include/rownorm.h"]:
        path = os.path.normpath(os.path.join(csrc, f))
        h.update(open(path, "rb").read())  # a missing file is an error, not a silent skip
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
    """S resident copies of one workload's inputs and outputs, with the buffers of both
    the trainable and the frozen backward (the frozen one passes null dW/dB)."""

    def __init__(self, wl, S, rn, torch):
        self.wl, self.S, self.rn, self.torch = wl, S, rn, torch
        base = workloads.generate(wl)
        dev = torch.device("cuda:0")
        self.eps, self.off = base["eps"], base["offset"]
        M, N = wl.M, wl.N
        ngr = 2 if wl.op == "layernorm" else 1
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
            d["dw"] = torch.empty(N, dtype=torch.float32, device=dev)
            d["db"] = torch.empty(N, dtype=torch.float32, device=dev) if wl.op == "layernorm" \
                else None
            # zero-filled once: the library's hand-over counters live at its start
            d["ws"] = rn.new_workspace(rn.workspace_bytes(M, N, ngr), dev)
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

    def bwd(self, s, trainable):
        d, rn, wl = self.sets[s], self.rn, self.wl
        dw = d["dw"] if trainable else None
        ws = d["ws"] if trainable else None
        if wl.op == "rmsnorm":
            rn.rmsnorm_bwd(d["dy"], d["x"], d["w"], self.eps, self.off, dx=d["dx"], dw=dw,
                           workspace=ws)
        elif wl.op == "layernorm":
            rn.layernorm_bwd(d["dy"], d["x"], d["w"], self.eps, dx=d["dx"], dw=dw,
                             db=d["db"] if trainable else None, workspace=ws)
        else:
            rn.fused_add_rmsnorm_bwd(d["dy"], d["ro"], d["w"], self.eps, self.off, d.get("dres"),
                                     dx=d["dx"], dw=dw, workspace=ws)

    def step(self, k, trainable):
        self.fwd(k % self.S)
        self.bwd((k + self.S // 2) % self.S, trainable)


MAX_SETS = 256


def n_sets(bytes_per_set: int) -> int:
    """Buffer sets to rotate through: more than three times the MALL in total, so every
    step reads data evicted from L2 and MALL.  Capped at MAX_SETS: a problem too small to
    reach that (a single decode row) is timed with its sets partly cache-resident."""
    s = 2
    while s * bytes_per_set < 3 * MALL_BYTES and s < MAX_SETS:
        s += 2
    return max(s, 4)


PROVIDERS = ("trainable", "frozen", "trainable_aa")


def capture(sets, K, trainable, torch):
    """A HIP graph of exactly K steps (the library's calls never allocate or
    synchronise, so they capture as they are)."""
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for k in range(K):
                sets.step(k, trainable)
    torch.cuda.synchronize()
    return g


def median(a):
    a = sorted(a)
    n = len(a)
    return a[n // 2] if n % 2 else 0.5 * (a[n // 2 - 1] + a[n // 2])


def time_rounds(sets, K, W, rounds, torch, seed=0, eager=False):
    """Per-step device time (us) of each provider: median over `rounds` rounds of one
    replay of each provider's K-step graph, providers in a shuffled order per round
    (eager: the K steps launched one by one instead, for profilers that count per
    dispatch).  Returns ({provider: median us/step}, {provider: [us/step per round]},
    wall seconds of the timed replays)."""
    for k in range(W):
        sets.step(k, True)
        sets.step(k, False)
    torch.cuda.synchronize()

    class Eager:
        def __init__(self, trainable):
            self.trainable = trainable

        def replay(self):
            for k in range(K):
                sets.step(k, self.trainable)

    graphs = {p: (Eager(p != "frozen") if eager else capture(sets, K, p != "frozen", torch))
              for p in PROVIDERS}
    for g in graphs.values():   # one untimed replay each
        g.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    rng = random.Random(seed)
    per = {p: [] for p in PROVIDERS}
    wall = 0.0
    for _ in range(rounds):
        order = list(PROVIDERS)
        rng.shuffle(order)
        for p in order:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            e0.record(st)
            graphs[p].replay()
            e1.record(st)
            torch.cuda.synchronize()
            wall += time.perf_counter() - t0
            per[p].append(e0.elapsed_time(e1) * 1e3 / K)
    del graphs
    return {p: median(v) for p, v in per.items()}, per, wall


def call_times(sets, n, trainable, torch):
    """Per-kernel and per-call device times (us): an eager pass of n steps queued behind
    a spin kernel (so the GPU runs them back to back).  The forward kernel and the
    backward's first kernel record dispatch events (instrumentation hook); the whole
    backward call (with parameter gradients: two kernels) is bracketed by HIP events on
    the launch stream."""
    rn = sets.rn
    st = torch.cuda.current_stream()
    mk = lambda: torch.cuda.Event(enable_timing=True)
    ev = [[mk() for _ in range(6)] for _ in range(n)]
    for e in (x for row in ev for x in row):
        e.record(st)                      # materialise the event handles
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2.4e9 * (0.002 + 40e-6 * n)))   # ~ 2 ms + 40 us per step
    try:
        for k in range(n):
            f0, f1, k0, k1, b0, b1 = ev[k]
            rn._set_timing_events(0, f0, f1)
            sets.fwd(k % sets.S)
            rn._set_timing_events(0, None, None)
            rn._set_timing_events(1, k0, k1)
            b0.record(st)
            sets.bwd((k + sets.S // 2) % sets.S, trainable)
            b1.record(st)
            rn._set_timing_events(1, None, None)
    finally:
        rn._set_timing_events(0, None, None)
        rn._set_timing_events(1, None, None)
    torch.cuda.synchronize()
    f = [ev[k][0].elapsed_time(ev[k][1]) * 1e3 for k in range(n)]
    k1 = [ev[k][2].elapsed_time(ev[k][3]) * 1e3 for k in range(n)]
    b = [ev[k][4].elapsed_time(ev[k][5]) * 1e3 for k in range(n)]
    return {"fwd_us_median": median(f), "fwd_us_mean": sum(f) / n,
            "bwd_kernel1_us_median": median(k1), "bwd_kernel1_us_mean": sum(k1) / n,
            "bwd_us_median": median(b), "bwd_us_mean": sum(b) / n}


def stream_ceiling(sets, n, torch) -> dict:
    """Context for the backward roofline: torch's own elementwise kernel moving the same
    row tensors as the backward (2 reads + 1 write; the fused add's 3 + 1), on the same
    rotating buffer sets, timed like the library's calls (events around each launch,
    queued behind a spin kernel).  No reduction, no fp64: what streaming alone reaches
    on this GPU for this size."""
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
    t = median([ev[k][0].elapsed_time(ev[k][1]) * 1e3 for k in range(n)])
    x = sets.sets[0]["x"]
    nbytes = x.numel() * x.element_size() * (4 if fused else 3)
    return {"op": "torch.addcmul, 3 reads + 1 write" if fused else "torch.mul, 2 reads + 1 write",
            "us_median": round(t, 3), "gbs": round(nbytes / (t * 1e-6) / 1e9, 1)}


# Threads the CPU baseline may use: one GPU's share of the host's cores on the GPU
# machines (16), or fewer when the process may use fewer.
CPU_SHARE = 16


def cpu_baseline(wl, budget_s: float, rows: int = 256) -> dict:
    """The oracle (numpy fp64, as it stands, never tuned) on a bounded sample of the
    workload's rows, forward + backward, on the host: every usable core (at most one
    GPU's share, CPU_SHARE threads), each thread running the same oracle calls on the
    sample, in rounds until `budget_s` has passed; then on one thread for another
    `budget_s`.  numpy releases the interpreter lock inside its array loops, so the
    threads run in parallel.  Each figure is the median round (repetition), as the
    sample's algorithmic bytes per second."""
    from concurrent.futures import ThreadPoolExecutor
    import numpy as np
    import oracle
    rows = min(wl.M, rows)
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

    usable = len(os.sched_getaffinity(0))
    cores = max(1, min(usable, CPU_SHARE))
    with ThreadPoolExecutor(max_workers=cores) as pool:
        list(pool.map(step, range(cores)))  # start the threads before timing
        per_all, n_all, el_all = timed(lambda: list(pool.map(step, range(cores))))
    per, n, el = timed(step)
    return {"value": round(cores * step_bytes / per_all / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{rows} of {wl.M} rows x {wl.N}, fwd+bwd (numpy fp64); {cores} threads "
                      f"each running it, median of {n_all} rounds in {el_all:.1f} s",
            "usable_cpus": usable,
            "thread_cap": f"at most {CPU_SHARE} threads (one GPU's share of the host)",
            "single_thread": {"value": round(step_bytes / per / 1e9, 4), "unit": "GB/s",
                              "cores": 1, "us_per_step_of_sample": round(per * 1e6, 1),
                              "sample": f"median of {n} repetitions in {el:.1f} s"},
            "cpu_model": _cpu_model()}


def _cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16


def distill_flops(wl, dx=True, dw=True) -> float:
    """Products of the fused linear JSD loss: student and teacher logits (2 B T V H
    each), dx = dz W and dW = dz^T x (2 B T V H each, when requested)."""
    one = 2.0 * wl.BT * wl.V * wl.H
    return one * (2 + int(dx) + int(dw))


def measure_distill(wl, rounds, torch, seed=1):
    """The distillation loss at one size: providers trainable (dx and dW), frozen (dx
    only: the student head frozen, [distill] Summary) and an identical trainable A/A
    duplicate, each call timed with HIP events, shuffled per round; medians in ms."""
    from normalization_row_wise_amd import distill
    t = workloads.generate_distill(wl)
    d = {k: (v.to("cuda:0") if v is not None else None) for k, v in t.items()}
    need = distill.workspace_bytes(wl.BT, wl.H, wl.Ht, wl.V, wl.chunk, True, True, True)
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda:0")
    dx = torch.empty(wl.BT, wl.H, dtype=torch.bfloat16, device="cuda:0")
    dw = torch.empty(wl.V, wl.H, dtype=torch.float32, device="cuda:0")

    def call(p):
        distill.fused_linear_jsd(d["xs"], d["ws"], d["xt"], d["wt"], d["bs"], d["bt"], wl.beta,
                                 wl.temperature, wl.chunk, dx=dx,
                                 dw=None if p == "frozen" else dw, db=None, workspace=ws)

    provs = ("trainable", "frozen", "trainable_aa")
    for p in provs:
        call(p)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    rng = random.Random(seed)
    per = {p: [] for p in provs}
    for _ in range(rounds):
        order = list(provs)
        rng.shuffle(order)
        for p in order:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(st)
            call(p)
            e1.record(st)
            torch.cuda.synchronize()
            per[p].append(e0.elapsed_time(e1))
    med = {p: median(v) for p, v in per.items()}
    del d, ws, dx, dw
    torch.cuda.empty_cache()
    ft, ff = distill_flops(wl, True, True), distill_flops(wl, True, False)
    return {"BT": wl.BT, "H": wl.H, "V": wl.V, "chunk": wl.chunk,
            "ms_per_call": {p: round(v, 3) for p, v in med.items()},
            "aa_delta_pct": round(100 * (med["trainable_aa"] / med["trainable"] - 1), 2),
            "frozen_saving_pct": round(100 * (1 - med["frozen"] / med["trainable"]), 1),
            "tflops": {"trainable": round(ft / (med["trainable"] * 1e-3) / 1e12, 1),
                       "frozen": round(ff / (med["frozen"] * 1e-3) / 1e12, 1)},
            "pct_of_bf16_mfma_peak": round(100 * ft / (med["trainable"] * 1e-3) / 1e12
                                           / MFMA_BF16_PEAK_TFLOPS, 2)}


# Configurations timed beside the headline, reported as extra keys of the same line.
EXTRA = ("layernorm_2048x4096_bf16", "fused_add_rmsnorm_2048x8192_bf16")


def measure(wl, K, W, rounds, rn, torch, event_steps, eager=False):
    """The protocol above on one workload: providers' median step times, A/A delta,
    per-call kernel times and the step's algorithmic GB/s."""
    probe = Sets(wl, 1, rn, torch)
    S = n_sets(probe.bytes_per_set)
    cold = S * probe.bytes_per_set >= 3 * MALL_BYTES
    del probe
    sets = Sets(wl, S, rn, torch)
    med, per, wall = time_rounds(sets, K, W, rounds, torch, eager=eager)
    ev_t = call_times(sets, event_steps, True, torch)
    ev_f = call_times(sets, event_steps, False, torch)
    abt, abf = alg_bytes(wl, True), alg_bytes(wl, False)
    out = {
        "sets": sets, "S": S, "cold": cold, "wall": wall, "per_round": per,
        "us_per_step": {p: round(med[p], 3) for p in PROVIDERS},
        "aa_delta_pct": round(100 * (med["trainable_aa"] / med["trainable"] - 1), 2),
        "gbs": abt["step"] / (med["trainable"] * 1e-6) / 1e9,
        "frozen_gbs": abf["step"] / (med["frozen"] * 1e-6) / 1e9,
        "calls": {"fwd_kernel_us": round(ev_t["fwd_us_median"], 3),
                  "bwd_trainable_kernel1_us": round(ev_t["bwd_kernel1_us_median"], 3),
                  "bwd_trainable_call_us": round(ev_t["bwd_us_median"], 3),
                  "bwd_frozen_kernel_us": round(ev_f["bwd_kernel1_us_median"], 3),
                  "bwd_frozen_call_us": round(ev_f["bwd_us_median"], 3)},
        "ev_t": ev_t, "ev_f": ev_f,
    }
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="steps per timed replay")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rounds", type=int, default=9)
    ap.add_argument("--config", default=workloads.RMS_8192x8192.name,
                    choices=sorted(workloads.BY_NAME))
    ap.add_argument("--no-extra", action="store_true", help="skip the extra configurations")
    ap.add_argument("--eager", action="store_true",
                    help="launch the timed steps one by one instead of graph replays (counter runs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--event-steps", type=int, default=100)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 3 plain device copies of MIB MiB (counter calibration)")
    ap.add_argument("--distill-only", action="store_true",
                    help="only time the distillation loss sizes (profiler runs); prints "
                         "{\"distill_jsd\": ...}")
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
    if args.steps < 1 or args.rounds < 1:
        print("--steps and --rounds must be at least 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import __graft_entry__
    __graft_entry__.ensure_built()
    import normalization_row_wise_amd as rn

    if args.distill_only:
        out = {dwl.name: measure_distill(dwl, args.rounds, torch) for dwl in workloads.DISTILL_CONFIGS}
        print(json.dumps({"distill_jsd": out}), flush=True)
        return

    wl = workloads.BY_NAME[args.config]
    m = measure(wl, args.steps, args.warmup, args.rounds, rn, torch, args.event_steps, args.eager)
    sets = m["sets"]
    abt = alg_bytes(wl, True)
    ceiling = stream_ceiling(sets, args.event_steps, torch) if "dres" in sets.sets[0] or \
        wl.op != "fused_add_rmsnorm" else None
    # dominant kernel: the trainable backward's first kernel (dx, partial rows of dW)
    k1_us = m["ev_t"]["bwd_kernel1_us_mean"]
    achieved = abt["bwd_stage1"] / (k1_us * 1e-6) / 1e9
    traffic = measured_traffic(wl.name, "bwd_stage1_trainable")
    del m["sets"], sets
    torch.cuda.empty_cache()

    extra = {}
    if not args.no_extra:
        for name in EXTRA:
            if name == wl.name:
                continue
            e = measure(workloads.BY_NAME[name], args.steps, args.warmup, args.rounds, rn, torch,
                        args.event_steps, args.eager)
            extra[name] = {
                "us_per_step": e["us_per_step"], "aa_delta_pct": e["aa_delta_pct"],
                "gbs": round(e["gbs"], 1), "pct_of_hbm_peak": round(100 * e["gbs"] / HBM_PEAK_GBS, 2),
                "frozen_gbs": round(e["frozen_gbs"], 1), "us_per_call": e["calls"]}
            del e["sets"], e
            torch.cuda.empty_cache()

    distill_lines = {}
    if not args.no_extra:
        for dwl in workloads.DISTILL_CONFIGS:
            distill_lines[dwl.name] = measure_distill(dwl, max(3, args.rounds // 2), torch)

    med = m["us_per_step"]
    line = {
        "metric": "achieved HBM GB/s (% of peak) & µs/call, bf16 norm fwd+bwd at M×N",
        "value": round(m["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(med["trainable"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # arithmetic: row sums, dx and LayerNorm y in fp64; RMSNorm y and the dW/dB
        # accumulation in fp32; storage (config.io) bf16
        "dtype": "f64+f32",
        "arithmetic": {"row_sums": "f64", "dx": "f64", "y": "f32 (RMSNorm), f64 (LayerNorm)",
                       "dW_dB": "f32", "storage": wl.io},
        "data": "synthetic (seeded CPU randn, no dataset)",
        "config": {"workload": wl.name, "op": wl.op, "M": wl.M, "N": wl.N, "io": wl.io,
                   "weight": wl.wt, "trainable_params": True,
                   "timing": f"median of {args.rounds} shuffled rounds of "
                             f"{'eager launches' if args.eager else 'HIP-graph replays'} of "
                             f"{args.steps} steps (providers trainable, frozen, trainable A/A)",
                   "buffer_sets": m["S"], "inputs_cold_in_mall": m["cold"]},
        "pct_of_hbm_peak": round(100 * m["gbs"] / HBM_PEAK_GBS, 2),
        "us_per_step": med,
        "aa_delta_pct": m["aa_delta_pct"],
        "frozen_gbs": round(m["frozen_gbs"], 1),
        "us_per_call": m["calls"],
        "timed_replays_wall_s": round(m["wall"], 4),
        "roofline": {"kernel": "bwd_kernel (stage 1: dx + dW partial rows)",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "alg_bytes_per_launch": abt["bwd_stage1"],
                     "avg_launch_us": round(k1_us, 3),
                     "stream_ceiling": ceiling},
        "extra_configs": extra,
        "distill_jsd": distill_lines,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
