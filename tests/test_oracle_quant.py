"""Pins of the oracle's MXFP4 quantiser and Smooth-QK application (CPU only).

The format is OCP MXFP4 (E2M1 elements, E8M0 scale per 32), the stated
stand-in for the HIF4 format the HiFA4 abstract names but does not define.
Pins:
  * hand-worked E2M1 roundings (tests/golden/e2m1_rounding.txt);
  * a sweep of fp32 inputs around every rounding boundary and across every
    exponent, against a brute-force nearest-value search written here;
  * hand-worked MX blocks (tests/golden/mx_blocks.txt), and under the
    no-clip exponent rule (tests/golden/mx_blocks_noclip.txt) with its
    characterisation as the smallest unsaturated exponent;
  * idempotence and exact round trip of on-grid blocks;
  * hand-worked Smooth-QK direction (Q * s, K / s) and byte layouts.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _parse_float(tok: str) -> float:
    return float.fromhex(tok) if "0x" in tok.lower() else float(tok)


def brute_force_e2m1(y: np.ndarray) -> np.ndarray:
    """Nearest E2M1 magnitude by exhaustive search; ties to the even code.

    Magnitudes above 6 are first clamped to 6 (the MX saturating conversion).
    """
    a = np.minimum(np.abs(y), 6.0)[..., None]
    dist = np.abs(a - MAG)                       # [..., 8]
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best
    # among equally near codes prefer an even code (mantissa bit 0)
    even_pref = np.where(cand, np.where(np.arange(8) % 2 == 0, 0, 1) * 16 + np.arange(8), 99)
    code = even_pref.argmin(axis=-1)
    return (code | np.where(np.signbit(y), 8, 0)).astype(np.uint8)


def test_e2m1_value_table():
    for c in range(16):
        want = MAG[c & 7] * (-1.0 if c & 8 else 1.0)
        assert oracle.e2m1_value(c) == want


def test_e2m1_golden():
    n = 0
    with open(os.path.join(GOLDEN, "e2m1_rounding.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tok = line.split()
            y, want = _parse_float(tok[0]), int(tok[1], 16)
            assert oracle.e2m1_encode(y) == want, (line, oracle.e2m1_encode(y))
            assert brute_force_e2m1(np.array([y]))[0] == want, line
            n += 1
    assert n >= 25


def _sweep_inputs() -> np.ndarray:
    bits = []
    # every fp32 within +-2^15 ulps of each grid value and midpoint
    for p in [0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0]:
        c = np.array([p], dtype=np.float32).view(np.uint32)[0]
        bits.append(np.arange(int(c) - 32768, int(c) + 32768, dtype=np.int64).astype(np.uint32))
    # every exponent and top-7 mantissa bits up to 8.0
    top = np.arange(0, 0x41000000 >> 16, dtype=np.uint32) << 16
    bits.append(top)
    rng = np.random.default_rng(7)
    bits.append(rng.integers(0, 0x41000000, size=1 << 20, dtype=np.uint32))
    b = np.concatenate(bits)
    b = np.concatenate([b, b | np.uint32(0x80000000)])
    return b.view(np.float32).astype(np.float64)


def test_e2m1_sweep_against_brute_force():
    y = _sweep_inputs()
    got = oracle.e2m1_encode_array(y)
    want = brute_force_e2m1(y)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(y[i], got[i], want[i]) for i in bad[:10]]


def _golden_blocks(fname="mx_blocks.txt"):
    out = []
    with open(os.path.join(GOLDEN, fname)) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, xs, sc, cs = [t.strip() for t in line.split("|")]
            x = np.zeros(32)
            for kv in xs.split():
                i, v = kv.split("=")
                x[int(i)] = _parse_float(v)
            codes = np.zeros(32, dtype=np.uint8)
            for kv in cs.split():
                i, v = kv.split("=")
                codes[int(i)] = int(v, 16)
            out.append((name, x, int(sc), codes))
    return out


@pytest.mark.parametrize("name,x,scale,codes", _golden_blocks(), ids=lambda v: v if isinstance(v, str) else "")
def test_mx_block_golden(name, x, scale, codes):
    got_codes, got_scale, deq = oracle.mx_block(x)
    assert got_scale == scale
    np.testing.assert_array_equal(got_codes, codes)
    # dequantised value = signed E2M1 value * 2^(scale - 127)
    want_deq = np.array([MAG[c & 7] * (-1 if c & 8 else 1) for c in codes]) * 2.0 ** (scale - 127)
    np.testing.assert_array_equal(deq, want_deq)


@pytest.mark.parametrize("name,x,scale,codes", _golden_blocks("mx_blocks_noclip.txt"),
                         ids=lambda v: v if isinstance(v, str) else "")
def test_mx_block_noclip_golden(name, x, scale, codes):
    got_codes, got_scale, deq = oracle.mx_block(x, rule=1)
    assert got_scale == scale
    np.testing.assert_array_equal(got_codes, codes)
    want_deq = np.array([MAG[c & 7] * (-1 if c & 8 else 1) for c in codes]) * 2.0 ** (scale - 127)
    np.testing.assert_array_equal(deq, want_deq)


def test_mx_block_noclip_is_the_smallest_unsaturated_exponent():
    """The no-clip exponent X1 is the smallest X >= the OCP exponent X0 with
    max|x| <= 6 * 2^X; then no element saturates and every element lies within
    2^X1 of its dequantised value (half the widest E2M1 gap, 4 -> 6).  Where
    X1 == X0 the codes are the OCP codes."""
    rng = np.random.default_rng(23)
    moved = 0
    for trial in range(3000):
        x = rng.standard_normal(32) * np.exp2(rng.integers(-60, 60))
        if trial % 3 == 0:  # put the block maximum near 6 * 2^k
            i = rng.integers(0, 32)
            x[i] = np.sign(x[i] or 1.0) * np.abs(x).max() * rng.uniform(1.0, 1.6)
        c0, s0, d0 = oracle.mx_block(x, rule=0)
        c1, s1, d1 = oracle.mx_block(x, rule=1)
        amax = np.abs(x).max()
        x1 = s1 - 127
        assert s1 - s0 in (0, 1)
        assert amax <= 6.0 * 2.0 ** x1
        if s1 > s0:
            moved += 1
            assert amax > 6.0 * 2.0 ** (s0 - 127)
        else:
            np.testing.assert_array_equal(c1, c0)
        assert np.all(np.abs(d1 - x) <= 2.0 ** x1)
        np.testing.assert_array_equal(c1 & 7, brute_force_e2m1(x / 2.0 ** x1) & 7)
    assert moved > 300
    # the OCP rule does saturate such a block: 7.9 -> 6
    _, s, d = oracle.mx_block(np.array([7.9]), rule=0)
    assert s == 127 and d[0] == 6.0


def test_mx_block_idempotent_and_on_grid_round_trip():
    rng = np.random.default_rng(11)
    for trial in range(2000):
        x = rng.standard_normal(32) * np.exp2(rng.integers(-40, 40))
        if trial % 7 == 0:
            x[rng.integers(0, 32, size=5)] = 0.0
        c1, s1, d1 = oracle.mx_block(x)
        c2, s2, d2 = oracle.mx_block(d1)
        assert s1 == s2
        np.testing.assert_array_equal(c1 & 7, c2 & 7)
        np.testing.assert_array_equal(d1, d2)
    # blocks already on the grid (largest magnitude code 4.0 or 6.0) round-trip exactly
    for _ in range(500):
        e = int(rng.integers(-100, 100))
        codes = rng.integers(0, 16, size=32).astype(np.uint8)
        codes[rng.integers(0, 32)] = rng.choice([6, 7, 14, 15])
        vals = np.array([MAG[c & 7] * (-1 if c & 8 else 1) for c in codes]) * 2.0 ** e
        # the largest code decides the exponent: 4.0 -> e, 6.0 -> e
        c, s, d = oracle.mx_block(vals)
        assert s == e + 127
        np.testing.assert_array_equal(d, vals)


def test_quantize_rows_layout_and_smooth_direction():
    d = 64
    x = np.ones((1, 1, 1, d), dtype=np.float32)
    x[0, 0, 0, 33] = -3.0
    s = np.ones((1, d), dtype=np.float32)
    s[0, 0] = 4.0
    # queries: x * s -> channel 0 = 4; block 0 amax 4 -> exponent 0 (byte 127):
    # codes 4.0 -> 0x6, 1.0 -> 0x2.  Block 1 amax 3 -> exponent -1 (byte 126):
    # 1.0 -> 2.0 -> 0x4, -3 -> -6 -> 0xf.
    codes, scales, deq = oracle.quantize_rows(x, s, divide=False)
    assert list(scales[0, 0, 0]) == [127, 126]
    assert codes[0, 0, 0, 0] == 0x26          # element 0 low nibble, element 1 high nibble
    assert codes[0, 0, 0, 1] == 0x22
    assert codes[0, 0, 0, 16] == 0xF4         # elements 32 (1.0 -> 0x4) and 33 (-3 -> 0xf)
    assert deq[0, 0, 0, 0] == 4.0 and deq[0, 0, 0, 33] == -3.0
    # keys: x / s -> channel 0 = 0.25; block 0 amax 1 -> exponent -2 (byte 125):
    # 0.25 -> 1.0 -> 0x2, 1.0 -> 4.0 -> 0x6.
    codes, scales, deq = oracle.quantize_rows(x, s, divide=True)
    assert scales[0, 0, 0, 0] == 125
    assert codes[0, 0, 0, 0] == 0x62
    assert deq[0, 0, 0, 0] == 0.25


def test_quantize_rows_gqa_smooth_rows_and_capacity():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 4, 5, 32)).astype(np.float32)
    s = np.exp2(rng.integers(-3, 4, size=(2, 32))).astype(np.float32)   # powers of two: exact
    codes, scales, deq = oracle.quantize_rows(x, s, divide=False, cap=7)
    assert codes.shape == (2, 4, 7, 16) and scales.shape == (2, 4, 7, 1)
    # head h uses smooth row h // (H / Hs)
    codes0, scales0, _ = oracle.quantize_rows(x * s[[0, 0, 1, 1]][None, :, None, :], None,
                                              divide=False)
    np.testing.assert_array_equal(codes[:, :, :5], codes0)
    np.testing.assert_array_equal(scales[:, :, :5], scales0)
    assert not codes[:, :, 5:].any()
    # with quantise=False the smoothed fp32 values come back unquantised
    _, _, plain = oracle.quantize_rows(x, s, divide=True, quantise=False)
    np.testing.assert_array_equal(plain, (x / s[[0, 0, 1, 1]][None, :, None, :]).astype(np.float64))


def test_quantize_v_layout_tail_block():
    S, d = 40, 2
    x = np.zeros((1, 1, S, d), dtype=np.float32)
    x[0, 0, :, 0] = 1.0
    x[0, 0, 3, 0] = 2.0            # block 0 of channel 0: amax 2 -> exponent -1
    x[0, 0, 32:, 1] = 0.5          # tail block (tokens 32..39) of channel 1
    x[0, 0, 39, 1] = -1.5
    codes, scales, deq = oracle.quantize_v(x)
    assert codes.shape == (1, 1, 2, 2, 16)
    assert scales[0, 0, 0, 0] == 126 and scales[0, 0, 0, 1] == 0
    # channel 0, block 0: tokens 0,1 -> 1.0/2^-1 = 2.0 -> 0x4 each; token 3 -> 4.0 -> 0x6
    assert codes[0, 0, 0, 0, 0] == 0x44 and codes[0, 0, 0, 0, 1] == 0x64
    # tail block of channel 1: amax over the 8 valid tokens = 1.5 -> exponent -2 (byte 125)
    assert scales[0, 0, 1, 1] == 125
    assert codes[0, 0, 1, 1, 0] == 0x44      # 0.5 * 4 = 2.0 -> 0x4
    assert codes[0, 0, 1, 1, 3] == 0xF4      # token 39 (high nibble of byte 3): -6 -> 0xf
    assert not codes[0, 0, 1, 1, 4:].any()   # padding tokens 40..63 are zero
    # tail block of channel 0: amax over tokens 32..39 only (all 1.0), not the 2.0 at token 3
    assert scales[0, 0, 1, 0] == 125
    assert codes[0, 0, 1, 0, 0] == 0x66 and not codes[0, 0, 1, 0, 4:].any()
    np.testing.assert_array_equal(deq[0, 0, 39], [1.0, -1.5])
