"""Pins for the oracle's direct fp64 -> bf16 / fp16 / fp32 rounder.

Pinned against: the page's worked rounding example, torch's own float32 -> bf16 and
float32 -> fp16 casts (an independent RNE implementation) over every tie and near-tie
of every finite encoding, random float32 bit patterns, and hand-derived cases where a
value that float32 cannot hold must not be rounded twice.
"""
import numpy as np
import pytest
import torch

from oracle import from_bits, round_to, to_bits, ulp_distance
from tests.golden import load

TD = {"bf16": torch.bfloat16, "fp16": torch.float16}


def torch_round(v32: np.ndarray, dtype: str) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32))
    return t.to(TD[dtype]).double().numpy()


def same(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return np.all(both_nan | eq)


def test_worked_example_offset_sum():
    g = load("gemma_offset_sum.txt")
    exact = g["w_bf16"] + g["offset"]
    assert round_to(exact, "fp32") == g["sum_fp32"]
    assert round_to(exact, "bf16") == g["sum_bf16"]
    # ties-away would have given the upper neighbour, so this pins ties-to-even
    assert round_to(exact, "bf16") != 1.0078125


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_every_tie_and_near_tie_matches_torch(dtype):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = from_bits(bits, dtype)
    ok = np.isfinite(v)
    v = v[ok]
    nxt = from_bits((bits[ok].astype(np.uint32) + 1).astype(np.uint16), dtype)
    # stay within one sign: stepping the bit pattern of the largest positive finite
    # value gives +inf, of -0 gives the smallest negative subnormal, which is fine
    mid = np.where(np.isfinite(nxt), (v + nxt) / 2, v)      # exact in fp32 (one more bit)
    cand = [v, mid]
    m32 = mid.astype(np.float32)
    cand.append(np.nextafter(m32, np.float32(np.inf)).astype(np.float64))
    cand.append(np.nextafter(m32, np.float32(-np.inf)).astype(np.float64))
    for c in cand:
        c32 = c.astype(np.float32)
        assert np.all(c32.astype(np.float64) == c)            # all candidates are fp32 values
        assert same(round_to(c, dtype), torch_round(c32, dtype))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_random_fp32_patterns_match_torch(dtype):
    rng = np.random.default_rng(1234)
    u = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    v32 = u.view(np.float32)
    v32 = v32[~np.isnan(v32)]
    assert same(round_to(v32.astype(np.float64), dtype), torch_round(v32, dtype))


def test_fp32_target_matches_numpy_cast():
    rng = np.random.default_rng(7)
    v = rng.standard_normal(1_000_000) * np.exp2(rng.integers(-140, 120, 1_000_000))
    # numpy's float64 -> float32 cast is a single IEEE round-to-nearest-even
    assert same(round_to(v, "fp32"), v.astype(np.float32).astype(np.float64))


def test_no_double_rounding_for_values_float32_cannot_hold():
    # 1 + 2^-8 + 2^-40 is just above the bf16 tie between 1 and 1 + 2^-7; float32 would
    # first round it onto the tie and then to even (1.0).  Direct rounding goes up.
    just_above = 1.0 + 2.0**-8 + 2.0**-40
    assert round_to(just_above, "bf16") == 1.0078125
    assert torch.tensor(just_above, dtype=torch.float64).to(torch.bfloat16).item() == 1.0
    assert round_to(1.0 + 2.0**-8 - 2.0**-40, "bf16") == 1.0
    assert round_to(-(1.0 + 2.0**-8 + 2.0**-40), "bf16") == -1.0078125
    assert round_to(1.0 + 2.0**-11 + 2.0**-40, "fp16") == 1.0 + 2.0**-10
    assert round_to(1.0 + 2.0**-24 + 2.0**-45, "fp32") == 1.0 + 2.0**-23
    # an odd neighbour below a tie: 1 + 3*2^-8 is the tie between 1 + 2^-7 (odd) and
    # 1 + 2^-6 (even), so it rounds up; a hair below it rounds down
    assert round_to(1.0 + 3 * 2.0**-8, "bf16") == 1.0 + 2.0**-6
    assert round_to(1.0 + 3 * 2.0**-8 - 2.0**-45, "bf16") == 1.0 + 2.0**-7


def test_special_values_and_overflow():
    for dt in ("bf16", "fp16", "fp32"):
        r = round_to(np.array([0.0, -0.0, np.inf, -np.inf, np.nan]), dt)
        assert r[0] == 0 and not np.signbit(r[0])
        assert r[1] == 0 and np.signbit(r[1])
        assert r[2] == np.inf and r[3] == -np.inf and np.isnan(r[4])
    bmax = float.fromhex("0x1.fep127")
    half = 2.0**119                    # half a bf16 spacing at the top binade
    assert round_to(bmax + half - 2.0**90, "bf16") == bmax
    assert round_to(bmax + half, "bf16") == np.inf          # tie goes to the even "2^128"
    assert round_to(65504.0 + 15.99, "fp16") == 65504.0
    assert round_to(65520.0, "fp16") == np.inf
    # subnormals: smallest bf16 subnormal is 2^-133, fp16 is 2^-24
    assert round_to(2.0**-134, "bf16") == 0.0                # tie with 0 -> even (0)
    assert round_to(2.0**-134 * 1.5, "bf16") == 2.0**-133
    assert round_to(2.0**-25 * 3, "fp16") == 2.0**-23        # 1.5 * 2^-24 -> tie -> even (2)
    assert round_to(-(2.0**-26), "fp16") == 0.0 and np.signbit(round_to(-(2.0**-26), "fp16"))


def test_bits_roundtrip_and_ulp_distance():
    v = np.array([1.0, -2.5, 3.015625, 0.0, -0.0])
    for dt in ("bf16", "fp16", "fp32"):
        assert same(from_bits(to_bits(v, dt), dt), v)
    a = to_bits(np.array([0.0, 1.0, 2.0**-133]), "bf16")
    b = to_bits(np.array([-0.0, 1.0078125, -(2.0**-133)]), "bf16")
    assert list(ulp_distance(a, b, "bf16")) == [0, 1, 2]
    a = to_bits(np.array([1.0]), "fp32")
    b = to_bits(np.array([np.nextafter(np.float32(1), np.float32(2))]), "fp32")
    assert ulp_distance(a, b, "fp32")[0] == 1
