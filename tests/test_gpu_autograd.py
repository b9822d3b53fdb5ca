"""GPU: the autograd layer over the library.  Gradients through torch.autograd match the
fp64 oracle; a parameter with requires_grad=False gets no gradient and leaves dx bit for
bit unchanged (the frozen kernel instance runs); inputs with leading dimensions and
non-contiguous gradients are handled.

Each case prints what it is before touching the GPU.
"""
import pytest
import torch

import oracle
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


def _f64(t):
    return workloads.as_f64(t.reshape(-1, t.shape[-1]))


def _io_ok(got, ref, io="bf16"):
    rep = gp.io_report(got.reshape(-1, got.shape[-1]).cpu(), ref, io)
    assert gp.io_ok(rep, io), rep


def _grad_ok(got, ref):
    assert gp.f32_report(got.float().cpu(), ref) <= 5e-3  # gradient returned in bf16


@pytest.mark.parametrize("frozen", [False, True], ids=["trainable", "frozen"])
def test_rmsnorm_module(frozen):
    from normalization_row_wise_amd.autograd import RMSNorm
    _say("autograd rmsnorm", "frozen" if frozen else "trainable")
    g = torch.Generator().manual_seed(5)
    B, S, N = 3, 37, 4096
    x = torch.randn(B, S, N, generator=g).to(torch.bfloat16)
    dy = torch.randn(B, S, N, generator=g).to(torch.bfloat16)
    m = RMSNorm(N, eps=1e-6, offset=1.0, device=gp.dev())
    with torch.no_grad():
        m.weight.copy_((torch.randn(N, generator=g) * 0.01).to(torch.bfloat16))
    m.weight.requires_grad_(not frozen)
    xd = x.to(gp.dev()).requires_grad_(True)
    y = m(xd)
    y.backward(dy.to(gp.dev()))
    torch.cuda.synchronize()
    w64 = workloads.as_f64(m.weight.detach())
    ry, _ = oracle.rmsnorm_fwd(_f64(x), w64, 1e-6, 1.0)
    rdx, rdw = oracle.rmsnorm_bwd(_f64(dy), _f64(x), w64, 1e-6, 1.0)
    _io_ok(y.detach(), ry)
    _io_ok(xd.grad, rdx)
    if frozen:
        assert m.weight.grad is None
    else:
        assert m.weight.grad.dtype == torch.bfloat16
        _grad_ok(m.weight.grad, rdw)


def test_frozen_weight_leaves_dx_bit_identical():
    from normalization_row_wise_amd.autograd import LayerNorm
    _say("autograd layernorm frozen vs trainable dx")
    g = torch.Generator().manual_seed(6)
    x = torch.randn(513, 2048, generator=g).to(torch.bfloat16).to(gp.dev())
    dy = torch.randn(513, 2048, generator=g).to(torch.bfloat16).to(gp.dev())
    grads = []
    for train_w, train_b in ((True, True), (False, False), (True, False), (False, True)):
        m = LayerNorm(2048, device=gp.dev())
        m.weight.requires_grad_(train_w)
        m.bias.requires_grad_(train_b)
        xd = x.clone().requires_grad_(True)
        m(xd).backward(dy)
        torch.cuda.synchronize()
        assert (m.weight.grad is not None) == train_w
        assert (m.bias.grad is not None) == train_b
        grads.append(xd.grad.view(torch.int16).clone())
    for gr in grads[1:]:
        assert torch.equal(gr, grads[0])


def test_layernorm_module_against_oracle():
    from normalization_row_wise_amd.autograd import LayerNorm
    _say("autograd layernorm")
    g = torch.Generator().manual_seed(7)
    B, S, N = 2, 100, 1000              # N not a multiple of 8: element accesses
    x = torch.randn(B, S, N, generator=g).to(torch.bfloat16)
    dy = torch.randn(B, S, N, generator=g).to(torch.bfloat16)
    m = LayerNorm(N, eps=1e-5, device=gp.dev())
    with torch.no_grad():
        m.weight.copy_((1 + 0.1 * torch.randn(N, generator=g)).to(torch.bfloat16))
        m.bias.copy_((0.1 * torch.randn(N, generator=g)).to(torch.bfloat16))
    xd = x.to(gp.dev()).requires_grad_(True)
    y = m(xd)
    y.backward(dy.to(gp.dev()))
    torch.cuda.synchronize()
    w64, b64 = workloads.as_f64(m.weight.detach()), workloads.as_f64(m.bias.detach())
    ry, _, _ = oracle.layernorm_fwd(_f64(x), w64, b64, 1e-5)
    rdx, rdw, rdb = oracle.layernorm_bwd(_f64(dy), _f64(x), w64, 1e-5)
    _io_ok(y.detach(), ry)
    _io_ok(xd.grad, rdx)
    _grad_ok(m.weight.grad, rdw)
    _grad_ok(m.bias.grad, rdb)


def test_fused_add_module_both_outputs_used():
    from normalization_row_wise_amd.autograd import FusedAddRMSNorm
    _say("autograd fused add")
    g = torch.Generator().manual_seed(8)
    B, S, N = 4, 64, 8192
    x = torch.randn(B, S, N, generator=g).to(torch.bfloat16)
    r = torch.randn(B, S, N, generator=g).to(torch.bfloat16)
    dy = torch.randn(B, S, N, generator=g).to(torch.bfloat16)
    dro = torch.randn(B, S, N, generator=g).to(torch.bfloat16)
    m = FusedAddRMSNorm(N, eps=1e-6, offset=1.0, device=gp.dev())
    with torch.no_grad():
        m.weight.copy_((torch.randn(N, generator=g) * 0.01).to(torch.bfloat16))
    xd = x.to(gp.dev()).requires_grad_(True)
    rd = r.to(gp.dev()).requires_grad_(True)
    y, ro = m(xd, rd)
    torch.autograd.backward([y, ro], [dy.to(gp.dev()), dro.to(gp.dev())])
    torch.cuda.synchronize()
    w64 = workloads.as_f64(m.weight.detach())
    ry, rro, _ = oracle.fused_add_rmsnorm_fwd(_f64(x), _f64(r), w64, 1e-6, 1.0, "bf16")
    rdx, rdw = oracle.fused_add_rmsnorm_bwd(_f64(dy), _f64(dro), rro, w64, 1e-6, 1.0)
    _io_ok(y.detach(), ry)
    _io_ok(ro.detach(), rro)
    _io_ok(xd.grad, rdx)
    assert torch.equal(xd.grad, rd.grad)
    _grad_ok(m.weight.grad, rdw)


def test_noncontiguous_gradient():
    from normalization_row_wise_amd.autograd import RMSNorm
    _say("autograd non-contiguous dy")
    g = torch.Generator().manual_seed(9)
    N = 512
    x = torch.randn(64, N, generator=g).to(torch.bfloat16).to(gp.dev())
    m = RMSNorm(N, device=gp.dev())
    xd = x.clone().requires_grad_(True)
    y = m(xd)
    big = torch.randn(N, 64, generator=g).to(torch.bfloat16).to(gp.dev())
    (y * big.t()).sum().backward()      # dy arrives as a transposed (strided) tensor
    xd2 = x.clone().requires_grad_(True)
    m(xd2).backward(big.t().contiguous())
    torch.cuda.synchronize()
    assert torch.equal(xd.grad.view(torch.int16), xd2.grad.view(torch.int16))


@pytest.mark.parametrize("frozen", [False, True], ids=["trainable", "frozen"])
def test_decode_row_module(frozen):
    """One token of a wide model (the split-row kernels): y, dx and dw against the
    oracle, with the weight trainable or frozen."""
    from normalization_row_wise_amd.autograd import RMSNorm
    _say("autograd decode row", "frozen" if frozen else "trainable")
    g = torch.Generator().manual_seed(10)
    N = 18432
    x = torch.randn(1, 1, N, generator=g).to(torch.bfloat16)
    dy = torch.randn(1, 1, N, generator=g).to(torch.bfloat16)
    m = RMSNorm(N, eps=1e-6, device=gp.dev(), dtype=torch.float32)
    with torch.no_grad():
        m.weight.copy_(1 + 0.1 * torch.randn(N, generator=g))
    m.weight.requires_grad_(not frozen)
    xd = x.to(gp.dev()).requires_grad_(True)
    y = m(xd)
    y.backward(dy.to(gp.dev()))
    torch.cuda.synchronize()
    w64 = workloads.as_f64(m.weight.detach())
    ry, _ = oracle.rmsnorm_fwd(_f64(x), w64, 1e-6, 0.0)
    rdx, rdw = oracle.rmsnorm_bwd(_f64(dy), _f64(x), w64, 1e-6, 0.0)
    _io_ok(y.detach(), ry)
    _io_ok(xd.grad, rdx)
    if frozen:
        assert m.weight.grad is None
    else:
        assert m.weight.grad.dtype == torch.float32
        assert gp.f32_report(m.weight.grad.cpu(), rdw) <= gp.REL_GRAD


@pytest.mark.parametrize("in_place", [False, True], ids=["out_of_place", "in_place"])
def test_page_call_signature(in_place):
    """The call of the Gemma page's reproduction, (x, w, eps, offset, casting_mode,
    in_place, row_mode), on its 128 x 4096 bf16 problem, against the oracle."""
    from normalization_row_wise_amd.autograd import RMSNormFunction
    _say("autograd page call", "in place" if in_place else "out of place")
    g = torch.Generator().manual_seed(42)
    x = torch.randn(128, 4096, generator=g).to(torch.bfloat16)
    w = (torch.randn(4096, generator=g) * 0.01).to(torch.bfloat16)
    dy = torch.randn(128, 4096, generator=g).to(torch.bfloat16)
    xd = x.to(gp.dev()).requires_grad_(True)
    wd = w.to(gp.dev()).requires_grad_(True)
    y = RMSNormFunction.apply(xd, wd, 1e-6, 1.0, "gemma", in_place, None)
    gx, gw = torch.autograd.grad(y, (xd, wd), dy.to(gp.dev()))
    torch.cuda.synchronize()
    w64 = workloads.as_f64(w)
    ry, _ = oracle.rmsnorm_fwd(_f64(x), w64, 1e-6, 1.0)
    rdx, rdw = oracle.rmsnorm_bwd(_f64(dy), _f64(x), w64, 1e-6, 1.0)
    _io_ok(y.detach(), ry)
    _io_ok(gx, rdx)
    _grad_ok(gw, rdw)
    with pytest.raises(ValueError):
        RMSNormFunction.apply(xd, wd, 1e-6, 1.0, "llama", False, None)


def test_gradient_broadcast_along_rows():
    """y.sum(0) sends the same gradient row to every row (a zero row stride): the binding
    copies it instead of handing overlapping rows to the kernels."""
    from normalization_row_wise_amd.autograd import LayerNorm
    _say("autograd broadcast gradient")
    g = torch.Generator().manual_seed(12)
    x = torch.randn(64, 1024, generator=g).to(torch.bfloat16).to(gp.dev())
    up = torch.randn(1024, generator=g).to(torch.bfloat16).to(gp.dev())
    m = LayerNorm(1024, device=gp.dev())
    xd = x.clone().requires_grad_(True)
    (m(xd).sum(0) * up).sum().backward()
    xd2 = x.clone().requires_grad_(True)
    m2 = LayerNorm(1024, device=gp.dev())
    m2(xd2).backward(up.expand(64, 1024).contiguous())
    torch.cuda.synchronize()
    assert torch.equal(xd.grad.view(torch.int16), xd2.grad.view(torch.int16))
    assert torch.equal(m.weight.grad, m2.weight.grad)
