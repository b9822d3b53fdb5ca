"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The C ABI sources are compiled for the host only (no device code) with both sanitizers
and linked, in place of the HIP runtime, with tests/abi_mock_hip.cpp (registration
accepted and ignored, launches checked against the hardware's limits and not run) and
tests/abi_sanitize_driver.cpp, which walks every entry point over a grid of valid
shapes, types and gradient selections and a set of invalid arguments.  The run exercises
the argument checks, the launch plans, the workspace layouts, the dispatch to kernel
instances and the launch sequences on the CPU; the sanitizers abort it on any memory or
undefined-behaviour error.  No GPU and no HIP runtime are used.
"""
import os
import re
import shlex
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "normalization_row_wise_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
SOURCES = ["rn_abi", "rn_fwd_rms", "rn_fwd_ln", "rn_fwd_fadd", "rn_bwd_rms", "rn_bwd_ln",
           "rn_bwd_fadd", "dl_abi"]
# host-only compilation; each sanitizer flag applies to the host pass
FLAGS = shlex.split("--offload-host-only -std=c++17 -O1 -g -fno-omit-frame-pointer "
                    "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                    "-Xclang -target-feature -Xclang -packed-fp32-ops")


# host compiler flags (no .hip file and no device code on these lines)
SAN = shlex.split("-fsanitize=address,undefined -fno-omit-frame-pointer")


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="hipcc not available")
def test_host_code_under_asan_and_ubsan(tmp_path):
    objs, procs = [], []
    for s in SOURCES:
        o = str(tmp_path / f"{s}.o")
        objs.append(o)
        procs.append(subprocess.Popen([HIPCC, "-x", "hip", *FLAGS, "-c", os.path.join(CSRC, f"{s}.hip"),
                                       "-o", o], stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
    drv = str(tmp_path / "driver.o")
    procs.append(subprocess.Popen([HIPCC, "-x", "hip", *FLAGS, "-c",
                                   os.path.join(ROOT, "tests", "abi_sanitize_driver.cpp"), "-o", drv],
                                  stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
    for p in procs:
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0, out.decode(errors="replace")[-3000:]
    # the host objects name the device binary each would embed; the mock ignores it
    names = set()
    for o in objs:
        nm = subprocess.run(["nm", "-u", o], stdout=subprocess.PIPE, check=True).stdout.decode()
        names.update(re.findall(r"\b(__hip_fatbin_[0-9a-f]+)\b", nm))
    stub = tmp_path / "fatbin_stubs.cpp"
    stub.write_text("".join(f'extern "C" const unsigned char {n}[16] = {{0}};\n' for n in sorted(names)))
    mock = str(tmp_path / "mock.o")
    for src, out in ((os.path.join(ROOT, "tests", "abi_mock_hip.cpp"), mock),
                     (str(stub), str(tmp_path / "stubs.o"))):
        r = subprocess.run([CLANG, "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__",
                            "-I/opt/rocm/include", *SAN, "-c", src, "-o", out],
                           stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=300)
        assert r.returncode == 0, r.stdout.decode(errors="replace")[-3000:]
    exe = str(tmp_path / "abi_sanitize")
    link = subprocess.run([CLANG, *SAN, *objs, drv, mock, str(tmp_path / "stubs.o"), "-o", exe],
                          stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=600)
    assert link.returncode == 0, link.stdout.decode(errors="replace")[-3000:]
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, env=env, timeout=600)
    text = r.stdout.decode(errors="replace")
    assert r.returncode == 0, text[-4000:]
    assert "runtime error" not in text and "AddressSanitizer" not in text, text[-4000:]
    assert " 0 bad launches, 0 failures" in text, text[-2000:]
    assert int(re.search(r"(\d+) launches", text).group(1)) > 1000, text[-2000:]
