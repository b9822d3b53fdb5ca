"""GPU: the same kernels under a broader calling contract.

* A captured HIP graph (torch.cuda.CUDAGraph) replayed with new values written into its
  input buffers: every replay must equal an eager call on the same values, bit for bit,
  and match the oracle.
* Two streams running different problems at once: results equal to running them alone.
* Strided rows and in-place backward over a matrix of row widths around the tile sizes.

Each case prints what it is before touching the GPU.
"""
import pytest
import torch

import workloads
from tests import gpu_parity as gp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import __graft_entry__
    __graft_entry__.ensure_built()


def _say(*a):
    print("[case]", *a, flush=True)


def _bits(t):
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16)


class Problem:
    """Static device buffers for one workload and the library calls on them."""

    def __init__(self, wl, trainable=True):
        import normalization_row_wise_amd as rn
        self.rn, self.wl, self.trainable = rn, wl, trainable
        t = workloads.generate(wl)
        self.eps, self.offset = t["eps"], t["offset"]
        self.inp = {k: v.to(gp.dev()) for k, v in t.items() if isinstance(v, torch.Tensor)}
        M, N = wl.M, wl.N
        like = self.inp["x"]
        f32 = dict(dtype=torch.float32, device=gp.dev())
        self.out = {"y": torch.empty_like(like), "dx": torch.empty_like(like),
                    "rstd": torch.empty(M, **f32)}
        if wl.op == "layernorm":
            self.out["mean"] = torch.empty(M, **f32)
        if wl.op == "fused_add_rmsnorm":
            self.out["residual_out"] = torch.empty_like(like)
        ngr = 0
        if trainable:
            self.out["dw"] = torch.empty(N, **f32)
            ngr = 1
            if wl.op == "layernorm":
                self.out["db"] = torch.empty(N, **f32)
                ngr = 2
        need = rn.workspace_bytes(M, N, ngr) if ngr else 0
        self.ws = rn.new_workspace(need, gp.dev()) if need else None

    def refill(self, seed):
        w = self.wl
        t = workloads.generate(workloads.small(w.op, w.M, w.N, w.io, w.wt, eps=w.eps,
                                               offset=w.offset, weight=w.weight, bias=w.bias,
                                               dres=w.dres, seed=seed))
        for k, v in self.inp.items():
            v.copy_(t[k].to(gp.dev()))
        return t

    def run(self, stream=None):
        rn, i, o, wl = self.rn, self.inp, self.out, self.wl
        dw = o.get("dw")
        if wl.op == "rmsnorm":
            rn.rmsnorm_fwd(i["x"], i["w"], self.eps, self.offset, y=o["y"], rstd=o["rstd"],
                           stream=stream)
            rn.rmsnorm_bwd(i["dy"], i["x"], i["w"], self.eps, self.offset, dx=o["dx"], dw=dw,
                           workspace=self.ws, stream=stream)
        elif wl.op == "layernorm":
            rn.layernorm_fwd(i["x"], i["w"], i.get("b"), self.eps, y=o["y"], mean=o["mean"],
                             rstd=o["rstd"], stream=stream)
            rn.layernorm_bwd(i["dy"], i["x"], i["w"], self.eps, dx=o["dx"], dw=dw,
                             db=o.get("db"), workspace=self.ws, stream=stream)
        else:
            rn.fused_add_rmsnorm_fwd(i["x"], i["residual"], i["w"], self.eps, self.offset,
                                     y=o["y"], residual_out=o["residual_out"], rstd=o["rstd"],
                                     stream=stream)
            rn.fused_add_rmsnorm_bwd(i["dy"], o["residual_out"], i["w"], self.eps, self.offset,
                                     i.get("dres"), dx=o["dx"], dw=dw, workspace=self.ws,
                                     stream=stream)

    def snapshot(self):
        return {k: v.clone() for k, v in self.out.items()}


GRAPH_CASES = [
    workloads.small("rmsnorm", 300, 4096, "bf16", offset=1.0, weight="gemma", seed=31),
    workloads.small("layernorm", 257, 4097, "bf16", seed=32),
    workloads.small("fused_add_rmsnorm", 130, 8192, "bf16", offset=1.0, weight="gemma", seed=33),
    workloads.small("rmsnorm", 64, 18432, "bf16", "fp32", seed=34),
    # split rows (a decode row; a small LayerNorm batch): several workgroups per row
    workloads.small("rmsnorm", 1, 18432, "bf16", "fp32", seed=35),
    workloads.small("layernorm", 3, 8192, "bf16", seed=36),
    # split rows whose workgroups are renumbered onto one XCD per row
    workloads.small("fused_add_rmsnorm", 32, 16384, "bf16", offset=1.0, weight="gemma", seed=37),
]


@pytest.mark.parametrize("trainable", [True, False], ids=["trainable", "frozen"])
@pytest.mark.parametrize("wl", GRAPH_CASES, ids=lambda c: c.name)
def test_graph_replay_with_new_inputs(wl, trainable):
    _say("graph", wl.name, "trainable" if trainable else "frozen")
    p = Problem(wl, trainable)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            p.run()                      # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        p.run()
    torch.cuda.synchronize()
    for k, seed in enumerate((101, 102, 103)):
        t = p.refill(seed)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replay = p.snapshot()
        p.run()                           # eager call on the same buffers and values
        torch.cuda.synchronize()
        eager = p.snapshot()
        for name in replay:
            assert torch.equal(_bits(replay[name]), _bits(eager[name])), (k, name)
        got = {kk: v.cpu() for kk, v in replay.items()}
        got.setdefault("dw", None)
        got.setdefault("db", None)
        o = gp.run_oracle(wl, t)
        if not trainable:
            o.pop("dw", None)
            o.pop("db", None)
        fails = gp.compare(wl, got, o)
        assert not fails, (k, fails)


def test_two_streams_at_once():
    _say("two streams")
    a = Problem(workloads.small("layernorm", 513, 4097, "bf16", seed=41))
    b = Problem(workloads.small("rmsnorm", 300, 8192, "fp16", offset=1.0, weight="gemma",
                                seed=42))
    a.run()
    b.run()
    torch.cuda.synchronize()
    ra, rb = a.snapshot(), b.snapshot()
    for v in list(a.out.values()) + list(b.out.values()):
        v.fill_(float("nan"))
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        a.run(stream=sa)
        b.run(stream=sb)
    torch.cuda.synchronize()
    for name in ra:
        assert torch.equal(_bits(a.out[name]), _bits(ra[name])), ("a", name)
    for name in rb:
        assert torch.equal(_bits(b.out[name]), _bits(rb[name])), ("b", name)


STRIDED_N = [512, 4095, 4097, 8191, 8193, 16383, 16385, 18432]


@pytest.mark.parametrize("n", STRIDED_N)
def test_strided_and_inplace_widths(n):
    import normalization_row_wise_amd as rn
    op = ["rmsnorm", "layernorm", "fused_add_rmsnorm"][STRIDED_N.index(n) % 3]
    off = 1.0 if op != "layernorm" else 0.0
    wl = workloads.small(op, 33, n, "bf16", offset=off, weight="gemma" if off else "unit",
                         seed=50 + n % 97)
    _say("strided+inplace", wl.name)
    t = workloads.generate(wl)
    o = gp.run_oracle(wl, t)
    M, N, pad = wl.M, n, 40
    td = torch.bfloat16

    def strided(src, lead):
        big = torch.zeros(M, N + pad, dtype=td, device=gp.dev())
        v = big[:, lead:lead + N]
        v.copy_(src.to(gp.dev()))
        return v

    x = strided(t["x"], 8)
    dy = strided(t["dy"], 16)
    w = t["w"].to(gp.dev())
    got = {}
    if op == "rmsnorm":
        got["y"], _ = rn.rmsnorm_fwd(x, w, t["eps"], t["offset"], y=strided(t["x"] * 0, 24))
        got["dx"], got["dw"] = rn.rmsnorm_bwd(dy, x, w, t["eps"], t["offset"], dx=dy)
    elif op == "layernorm":
        b = t["b"].to(gp.dev())
        got["y"], _, _ = rn.layernorm_fwd(x, w, b, t["eps"], y=strided(t["x"] * 0, 24))
        got["dx"], got["dw"], got["db"] = rn.layernorm_bwd(dy, x, w, t["eps"], dx=dy)
    else:
        res = strided(t["residual"], 32)
        got["y"], got["residual_out"], _ = rn.fused_add_rmsnorm_fwd(
            x, res, w, t["eps"], t["offset"], y=strided(t["x"] * 0, 24), residual_out=res)
        dres = strided(t["dres"], 8)
        got["dx"], got["dw"] = rn.fused_add_rmsnorm_bwd(dy, res, w, t["eps"], t["offset"], dres,
                                                        dx=dres)
        assert got["dx"].data_ptr() == dres.data_ptr()
    torch.cuda.synchronize()
    if op != "fused_add_rmsnorm":
        assert got["dx"].data_ptr() == dy.data_ptr()
    for k in ("y", "dx", "residual_out"):
        if k in got:
            rep = gp.io_report(got[k].cpu(), o[k], "bf16")
            assert gp.io_ok(rep, "bf16"), (k, rep)
    for k in ("dw", "db"):
        if k in got:
            assert gp.f32_report(got[k].cpu(), o[k]) <= gp.REL_GRAD, k
