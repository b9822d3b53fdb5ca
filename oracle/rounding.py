"""Round-to-nearest-even from fp64 to bf16 / fp16 / fp32, done directly (one rounding).

TEST INFRASTRUCTURE. This package is the correctness oracle. Only the test suite,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import it.
The HIP product path never imports or calls it.

Why a rounder of our own: every stored output of the method is one rounding of an
exact value to the I/O type.  Torch's double -> bfloat16 cast goes through float32
first, so it can round twice (a value just above a bf16 tie lands on the tie in
float32 and then goes to even).  Here the fp64 value is rounded once, straight to the
target grid, with numpy's ``rint`` (IEEE round-half-to-even) on an exact power-of-two
rescaling.

The rounding mode itself is fixed by the worked example on the page
"fix(cutedsl): fuse Gemma RMSNorm weight offset in FP32", Summary: the bf16 sum of
1 and 2^-8 is reported as 1.0.  1 + 2^-8 is exactly halfway between the bf16
neighbours 1.0 and 1.0078125; only ties-to-even gives 1.0 (ties-away would give
1.0078125).
"""
from __future__ import annotations

import numpy as np

# (significand bits incl. the implicit one, minimum normal exponent, largest finite value)
_FORMATS = {
    "bf16": (8, -126, float.fromhex("0x1.fep127")),
    "fp16": (11, -14, 65504.0),
    "fp32": (24, -126, float.fromhex("0x1.fffffep127")),
}

DTYPES = tuple(_FORMATS)


def round_to(v, dtype: str) -> np.ndarray:
    """Round fp64 values to the nearest ``dtype`` value, ties to even, in one step.

    Returns fp64 values that are exactly representable in ``dtype``.  Subnormals of
    the target are kept, values at or beyond the overflow threshold become +-inf,
    NaN stays NaN and the sign of zero is kept.
    """
    p, emin, vmax = _FORMATS[dtype]
    v = np.asarray(v, dtype=np.float64)
    out = v.copy()
    fin = np.isfinite(v) & (v != 0.0)
    a = v[fin]
    _, e = np.frexp(a)                       # a = m * 2**e, 0.5 <= |m| < 1
    lead = np.maximum(e - 1, emin)           # exponent of the leading bit (clamped: subnormals)
    q = np.ldexp(1.0, lead - (p - 1))        # spacing of the target grid at a
    r = np.rint(a / q) * q                   # a / q is exact: q is a power of two
    r = np.where(np.abs(r) > vmax, np.copysign(np.inf, a), r)
    out[fin] = r
    return out


def to_bits(v, dtype: str) -> np.ndarray:
    """Bit patterns of values already representable in ``dtype`` (uint16 / uint32)."""
    v = np.asarray(v, dtype=np.float64)
    if dtype == "bf16":
        return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    if dtype == "fp16":
        return v.astype(np.float16).view(np.uint16)
    if dtype == "fp32":
        return v.astype(np.float32).view(np.uint32)
    raise ValueError(dtype)


def from_bits(bits, dtype: str) -> np.ndarray:
    """Exact fp64 values of ``dtype`` bit patterns."""
    bits = np.asarray(bits)
    with np.errstate(invalid="ignore"):      # signalling-NaN patterns widen quietly
        if dtype == "bf16":
            return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        if dtype == "fp16":
            return bits.astype(np.uint16).view(np.float16).astype(np.float64)
        if dtype == "fp32":
            return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def ulp_distance(a_bits, b_bits, dtype: str) -> np.ndarray:
    """Number of representable values between two encodings (sign-magnitude ordinals).

    +0 and -0 are both ordinal 0.  Callers exclude NaN themselves.
    """
    width = 32 if dtype == "fp32" else 16
    sign = np.int64(1) << (width - 1)
    mag_mask = sign - 1

    def ordinal(b):
        b = np.asarray(b).astype(np.int64) & ((np.int64(1) << width) - 1)
        mag = b & mag_mask
        return np.where(b & sign, -mag, mag)

    return np.abs(ordinal(a_bits) - ordinal(b_bits))
