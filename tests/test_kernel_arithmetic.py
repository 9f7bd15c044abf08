"""Arithmetic identities the HIP kernels rely on, checked on the CPU.

The quantise kernel divides K by the smoothing factors (Smooth-QK: "HiFA4:
Training-Free 4-bit FlashAttention on Ascend HIF4 NPUs for LLM Inference",
Abstract) as RN32(x * RN64(1 / s)) with a per-workgroup table of double
reciprocals.  The codes must equal those of the fp32 division x / s (the oracle's
and the quantise kernel's definition), so this product must round to the same
float for every binary32 x and s: the double product is within 2^-52 of x / s,
and a quotient of two binary32 numbers is either exact or at least 2^-49 away
from the nearest binary32 rounding midpoint.
"""
import numpy as np


def _via_double_reciprocal(x, s):
    return (x.astype(np.float64) * (1.0 / np.float64(s))).astype(np.float32)


def _all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    return v[np.isfinite(v)]


def test_division_via_double_reciprocal_matches_fp32_division():
    rng = np.random.default_rng(11)
    xs = [_all_finite_bf16(),
          # fp32 values with full 24-bit significands (K after RoPE), all exponents
          (rng.standard_normal(200000) * np.exp2(rng.integers(-140, 120, 200000))).astype(np.float32)]
    # divisors: smoothing factors of every magnitude, powers of two, 24-bit
    # significands next to powers of two
    ss = np.concatenate([
        np.exp2(rng.uniform(-60, 60, 120)).astype(np.float32),
        np.exp2(np.arange(-20, 21, 5)).astype(np.float32),
        (np.float32(1) + np.float32(2.0 ** -23) * np.arange(1, 6, dtype=np.float32)),
        (np.float32(2) - np.float32(2.0 ** -23) * np.arange(1, 6, dtype=np.float32)),
        rng.uniform(0.05, 20, 60).astype(np.float32),
    ])
    with np.errstate(over="ignore", under="ignore", invalid="ignore", divide="ignore"):
        for s in ss:
            for x in xs:
                want = x / s
                got = _via_double_reciprocal(x, s)
                same = (want.view(np.uint32) == got.view(np.uint32)) | (np.isnan(want) & np.isnan(got))
                assert same.all(), (float(s), x[~same][:4], want[~same][:4], got[~same][:4])


def test_division_via_double_reciprocal_special_values():
    with np.errstate(over="ignore", under="ignore", invalid="ignore", divide="ignore"):
        x = np.array([0.0, -0.0, 1.0, -3.5, np.inf, -np.inf, np.nan, 3.4e38, 1e-45],
                     dtype=np.float32)
        for s in (np.float32(0.0), np.float32(np.inf), np.float32(1e-38), np.float32(3e38),
                  np.float32(0.7)):
            want = x / s
            got = _via_double_reciprocal(x, s)
            same = (want.view(np.uint32) == got.view(np.uint32)) | (np.isnan(want) & np.isnan(got))
            assert same.all(), (float(s), x[~same], want[~same], got[~same])
