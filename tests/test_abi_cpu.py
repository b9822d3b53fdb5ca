"""CPU-side checks of the C ABI: the library loads without a GPU, exports every
function include/rownorm.h declares, and rejects bad arguments with the documented
status codes before making any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rownorm.h")


@pytest.fixture(scope="module")
def rn():
    import __graft_entry__
    __graft_entry__.ensure_built()
    import normalization_row_wise_amd as rn
    return rn


DISTILL_HEADER = os.path.join(ROOT, "include", "distill.h")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"#[^\n]*", "", text)
    names = re.findall(r"\b([A-Za-z_]\w*)\s*\([^;{}]*\)\s*;", text)
    return sorted(set(names))


def test_header_declares_the_six_operations():
    names = declared_functions()
    for n in ("rmsnorm_fwd", "rmsnorm_bwd", "layernorm_fwd", "layernorm_bwd",
              "fused_add_rmsnorm_fwd", "fused_add_rmsnorm_bwd", "rn_bwd_workspace_bytes",
              "rn_status_str"):
        assert n in names


def test_library_exports_every_declared_symbol(rn):
    lib = ctypes.CDLL(rn.LIB_PATH)
    names = declared_functions() + declared_functions(DISTILL_HEADER)
    assert "fused_linear_jsd" in names and "fused_linear_jsd_workspace_bytes" in names
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_distill_argument_errors(rn):
    """fused_linear_jsd checks sizes, pointers, strides and the workspace before any HIP
    call; the workspace query is 0 for unsupported sizes and smaller for a frozen head."""
    L = rn.lib
    q = L.fused_linear_jsd_workspace_bytes
    assert q(4096, 4096, 4096, 128256, 1024, 1, 1, 1) > q(4096, 4096, 4096, 128256, 1024, 1, 0, 0)
    assert q(4096, 4096, 4096, 128256, 1024, 0, 0, 0) < q(4096, 4096, 4096, 128256, 1024, 1, 0, 0)
    assert q(4096, 4100, 4096, 128256, 1024, 1, 1, 1) == 0      # H not a multiple of 8
    assert q(-1, 64, 64, 100, 16, 1, 1, 1) == 0 and q(16, 64, 64, 0, 16, 1, 1, 1) == 0
    f = L.fused_linear_jsd
    A = ctypes.c_void_p(4096)
    need = q(16, 64, 64, 100, 8, 1, 1, 0)
    ok = dict(xs=A, ldxs=64, ws=A, bs=None, xt=A, ldxt=64, wt=A, bt=None, BT=16, H=64, Ht=64,
              V=100, beta=0.5, tau=1.0, chunk=8, loss=A, dx=A, lddx=64, dw=ctypes.c_void_p(8192),
              db=None, ws_buf=ctypes.c_void_p(1 << 20), ws_bytes=need, stream=None)

    def call(**over):
        a = {**ok, **over}
        return f(*a.values())
    assert call(H=60) == E_SHAPE
    assert call(beta=1.5) == E_SHAPE and call(tau=0.0) == E_SHAPE
    assert call(loss=None) == E_NULL and call(xs=None) == E_NULL
    assert call(db=A) == E_NULL                                # db without a bias
    assert call(ws_bytes=need - 1) == E_WS
    assert call(ws_buf=ctypes.c_void_p((1 << 20) + 16)) == E_WS   # not 256-byte aligned
    assert call(ldxs=60) == E_STRIDE and call(ldxs=68) == E_STRIDE
    assert call(xs=ctypes.c_void_p(4104)) == E_STRIDE        # not 16-byte aligned


RN_OK, E_NULL, E_SHAPE, E_DTYPE, E_STRIDE, E_WS, E_HIP, E_ALIAS, E_INT, E_SCRATCH = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9)
F32, F16, BF16 = 0, 1, 2
P = ctypes.c_void_p(4096)    # a non-null address that is never dereferenced
Q = ctypes.c_void_p(8192)
Rr = ctypes.c_void_p(12288)
S = ctypes.c_void_p(16384)


def test_status_strings(rn):
    for code in (RN_OK, E_NULL, E_SHAPE, E_DTYPE, E_STRIDE, E_WS, E_HIP, E_ALIAS, E_INT, E_SCRATCH):
        s = rn.lib.rn_status_str(code).decode()
        assert s and s != "unknown status"
    assert rn.lib.rn_status_str(42).decode() == "unknown status"


def test_workspace_query(rn):
    ws = rn.workspace_bytes
    assert ws(2048, 4096, 0) == 0              # frozen: nothing
    assert ws(0, 4096, 1) == 0                 # empty batch: nothing to stage
    one = ws(2048, 4096, 1)
    assert one > 0 and ws(2048, 4096, 2) == 2 * one
    assert one % 16 == 0 and one >= 4096 * 4
    assert one == 256 * 4096 * 4               # at most 256 partial rows of N fp32
    assert ws(3, 100, 1) == 3 * 128 * 4   # rows padded to 64 floats
    assert ws(8192, 8192, 1) >= ws(2048, 4096, 1)
    assert ws(-1, 4096, 1) == 0 and ws(4, 0, 1) == 0 and ws(4, 10**6, 1) == 0
    assert ws(4, 64, 3) == 0


def test_forward_argument_errors(rn):
    L = rn.lib
    f = L.rmsnorm_fwd
    assert f(P, 64, Q, Rr, 64, None, 0, 64, 1e-6, 0.0, BF16, BF16, None) == RN_OK   # M = 0: no-op
    assert f(P, 64, Q, Rr, 64, None, 4, 64, 1e-6, 0.0, 7, BF16, None) == E_DTYPE
    assert f(P, 64, Q, Rr, 64, None, 4, 64, 1e-6, 0.0, BF16, F16, None) == E_DTYPE  # mixed 16-bit
    assert f(P, 64, Q, Rr, 64, None, -1, 64, 1e-6, 0.0, BF16, BF16, None) == E_SHAPE
    assert f(P, 64, Q, Rr, 64, None, 4, 0, 1e-6, 0.0, BF16, BF16, None) == E_SHAPE
    assert f(P, 99999, Q, Rr, 99999, None, 4, 99999, 1e-6, 0.0, BF16, BF16, None) == E_SHAPE
    assert f(None, 64, Q, Rr, 64, None, 4, 64, 1e-6, 0.0, BF16, BF16, None) == E_NULL
    assert f(P, 64, None, Rr, 64, None, 4, 64, 1e-6, 0.0, BF16, BF16, None) == E_NULL
    assert f(P, 63, Q, Rr, 64, None, 4, 64, 1e-6, 0.0, BF16, BF16, None) == E_STRIDE
    assert f(P, 64, Q, Rr, 32, None, 4, 64, 1e-6, 0.0, BF16, BF16, None) == E_STRIDE
    g = L.layernorm_fwd
    assert g(P, 64, Q, None, Rr, 64, S, S, 4, 64, 1e-5, F32, F32, None) == E_ALIAS
    assert g(P, 64, None, None, Rr, 64, None, None, 4, 64, 1e-5, F32, F32, None) == E_NULL
    h = L.fused_add_rmsnorm_fwd
    assert h(P, 64, None, 64, Q, Rr, 64, S, 64, None, 4, 64, 1e-6, 1.0, BF16, BF16, None) == E_NULL
    assert h(P, 64, P, 64, Q, Rr, 64, Rr, 64, None, 4, 64, 1e-6, 1.0, BF16, BF16, None) == E_ALIAS
    assert h(P, 64, P, 16, Q, Rr, 64, S, 64, None, 4, 64, 1e-6, 1.0, BF16, BF16, None) == E_STRIDE


def test_backward_argument_errors(rn):
    L = rn.lib
    b = L.rmsnorm_bwd
    need = rn.workspace_bytes(4, 64, 1)
    # workspace missing or too small while dw is requested
    assert b(P, 64, Q, 64, Rr, S, 64, P, None, 0, 4, 64, 1e-6, 0.0, BF16, BF16, None) == E_WS
    assert b(P, 64, Q, 64, Rr, S, 64, P, Q, need - 4, 4, 64, 1e-6, 0.0, BF16, BF16, None) == E_WS
    assert b(P, 64, Q, 64, Rr, S, 64, P, ctypes.c_void_p(4100), need, 4, 64, 1e-6, 0.0, BF16,
             BF16, None) == E_WS                                   # misaligned workspace
    assert b(None, 64, Q, 64, Rr, S, 64, None, None, 0, 4, 64, 1e-6, 0.0, BF16, BF16, None) == E_NULL
    assert b(P, 64, Q, 64, Rr, None, 64, None, None, 0, 4, 64, 1e-6, 0.0, BF16, BF16, None) == E_NULL
    assert b(P, 8, Q, 64, Rr, S, 64, None, None, 0, 4, 64, 1e-6, 0.0, BF16, BF16, None) == E_STRIDE
    assert b(P, 64, Q, 64, Rr, S, 64, None, None, 0, 4, 64, 1e-6, 0.0, F16, BF16, None) == E_DTYPE
    ln = L.layernorm_bwd
    assert ln(P, 64, Q, 64, Rr, S, 64, P, P, Q, 1 << 20, 4, 64, 1e-5, F32, F32, None) == E_ALIAS
    need2 = rn.workspace_bytes(4, 64, 2)
    assert ln(P, 64, Q, 64, Rr, S, 64, P, Q, Rr, need2 - 16, 4, 64, 1e-5, F32, F32, None) == E_WS
    fa = L.fused_add_rmsnorm_bwd
    assert fa(P, 64, None, 0, None, 64, Rr, S, 64, None, None, 0, 4, 64, 1e-6, 1.0, BF16, BF16,
              None) == E_NULL                                      # residual_out missing
    assert fa(P, 64, Q, 8, Q, 64, Rr, S, 64, None, None, 0, 4, 64, 1e-6, 1.0, BF16, BF16,
              None) == E_STRIDE                                    # dres_out stride


def test_noalloc_refuses_before_any_hip_call(rn):
    """rmsnorm_bwd_noalloc checks the shape and its fixed scratch (8 MiB of partial rows)
    before touching the GPU: these return without a device present."""
    f = rn.lib.rmsnorm_bwd_noalloc
    assert f(P, 16384, Q, 16384, Rr, S, 16384, P, 4096, 16384, 1e-6, 0.0, BF16, BF16,
             None) == E_SCRATCH                                   # 256 x 64 KiB partial rows
    assert f(P, 64, Q, 64, Rr, S, 64, P, -1, 64, 1e-6, 0.0, BF16, BF16, None) == E_SHAPE
    assert f(P, 64, Q, 64, Rr, S, 64, P, 4, 99999, 1e-6, 0.0, BF16, BF16, None) == E_SHAPE
    assert rn.workspace_bytes(8192, 8192, 1) <= 8 << 20 < rn.workspace_bytes(4096, 16384, 1)


def test_no_process_wide_tuning_state(rn):
    """The product ABI holds no tuning state: no launch-shape override exists, and the
    one instrumentation hook (dispatch timing events, per calling thread) is declared
    only in the internal instrumentation header, not in include/rownorm.h."""
    lib = ctypes.CDLL(rn.LIB_PATH)
    assert not hasattr(lib, "rn_set_launch_override")
    assert "rn_set_timing_events" not in declared_functions()
    internal = open(os.path.join(ROOT, "normalization_row_wise_amd", "csrc",
                                 "rn_instrument.h")).read()
    assert "int rn_set_timing_events(" in internal and "thread" in internal
    src = open(os.path.join(ROOT, "normalization_row_wise_amd", "csrc", "rn_abi.hip")).read()
    assert "thread_local hipEvent_t t_timing" in src
    assert lib.rn_set_timing_events(2, None, None) == E_SHAPE
    assert lib.rn_set_timing_events(0, None, None) == RN_OK


def test_binding_refuses_host_tensors(rn):
    """A host address handed to a kernel would fault the GPU: the binding refuses CPU
    tensors before anything reaches the library."""
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    w = torch.ones(64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        rn.rmsnorm_fwd(x, w)
    with pytest.raises(ValueError, match="GPU tensor"):
        rn.layernorm_bwd(x, x, w)
    with pytest.raises(ValueError, match="GPU tensor"):
        rn.fused_add_rmsnorm_fwd(x, x, w)


def test_missing_library_raises(rn, tmp_path):
    """No CPU fallback: loading from a path with no built library raises ImportError."""
    with pytest.raises(ImportError, match="no CPU fallback"):
        rn.load_library(str(tmp_path / "librownorm.so"))


def test_product_path_never_touches_the_oracle():
    """The package and its C sources name no oracle module: the oracle is test
    infrastructure only."""
    pkg = os.path.join(ROOT, "normalization_row_wise_amd")
    offenders = []
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                if re.search(r"^\s*(import|from)\s+oracle\b|oracle/|\"oracle\"", src, re.M):
                    offenders.append(f)
    assert offenders == []
