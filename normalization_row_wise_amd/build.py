"""Build librownorm.so (HIP, gfx950) in-tree with hipcc.

Usage: python normalization_row_wise_amd/build.py   (or load this file and call build();
importing the package itself requires the built library).
Every .hip file under csrc/ is compiled to an object in parallel, then linked into
normalization_row_wise_amd/librownorm.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.environ.get("RN_BUILD_OUT", os.path.join(HERE, "librownorm.so"))
BUILD_DIR = os.environ.get("RN_BUILD_DIR", os.path.join(HERE, "_build"))
ARCH = os.environ.get("RN_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no implicit fma contraction: the source states every fma it wants, so the
    # frozen and trainable backward instances compute dx with the same operations
    "-ffp-contract=off",
    # keep the compiler from emitting packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    *os.environ.get("RN_EXTRA_FLAGS", "").split(),
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(src: str, obj: str) -> str:
    cmd = [_hipcc(), *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every kernel source and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [os.path.join(BUILD_DIR, f[:-4] + ".o") for f in srcs]
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_compile, os.path.join(CSRC, s), o) for s, o in zip(srcs, objs)]
        for f in futs:
            f.result()
            if verbose:
                print("built", f.result(), flush=True)
    tmp = OUT + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print("linked", OUT, flush=True)
    return OUT


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
