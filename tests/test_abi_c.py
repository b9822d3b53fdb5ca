"""The public headers as a C program sees them: tests/abi_c_client.c is compiled as C11
with every warning an error, linked against the built library and run (no GPU: it makes
only the calls that return before any HIP call).  It binds every entry point to a
pointer of its declared type; this test also checks that it names every function the
headers declare."""
import os
import re
import shutil
import subprocess

import pytest

from tests.test_abi_cpu import DISTILL_HEADER, HEADER, ROOT, declared_functions

CLIENT = os.path.join(ROOT, "tests", "abi_c_client.c")


@pytest.fixture(scope="module")
def libdir():
    import __graft_entry__
    __graft_entry__.ensure_built()
    import normalization_row_wise_amd as rn
    return os.path.dirname(rn.LIB_PATH)


def test_client_binds_every_declared_function():
    src = open(CLIENT).read()
    names = declared_functions(HEADER) + declared_functions(DISTILL_HEADER)
    missing = [n for n in names if not re.search(r"=\s*" + n + r"\s*;", src)]
    assert not missing, missing


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_headers_compile_link_and_run_as_c(libdir, tmp_path):
    exe = str(tmp_path / "abi_c_client")
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I/opt/rocm/include", CLIENT,
           "-L" + libdir, "-lrownorm", "-Wl,-rpath," + libdir, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
