"""Pins for the oracle's RoPE and Smooth-QK calibration (CPU only).

Each check fixes something the definitions imply without retyping them: the
identity and quarter-turn rotations are exact, the pair norm is preserved, the
table row used is the token's position, a rotation followed by its inverse
returns the input; the calibration reproduces hand-worked ratios, takes the
query maximum over exactly the heads of a group, and equalises the smoothed
maxima at alpha = 1/2.
"""
import numpy as np
import pytest

import oracle


def _tables(n_pos, half, ang):
    return (np.cos(ang).astype(np.float32) * np.ones((n_pos, half), np.float32),
            np.sin(ang).astype(np.float32) * np.ones((n_pos, half), np.float32))


def test_rope_identity_and_quarter_turn_are_exact():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 3, 5, 8)).astype(np.float32)
    c, s = np.ones((5, 4), np.float32), np.zeros((5, 4), np.float32)
    np.testing.assert_array_equal(oracle.rope_rows(x, c, s), x)
    # cos 0, sin 1: (a, b) -> (-b, a) on the pair (j, j + d/2)
    out = oracle.rope_rows(x, np.zeros((5, 4), np.float32), np.ones((5, 4), np.float32))
    np.testing.assert_array_equal(out[..., :4], -x[..., 4:])
    np.testing.assert_array_equal(out[..., 4:], x[..., :4])


def test_rope_uses_the_tokens_position_row():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, 2, 6, 4)).astype(np.float32)
    n_pos, pos0 = 20, 7
    c, s = np.ones((n_pos, 2), np.float32), np.zeros((n_pos, 2), np.float32)
    c[pos0 + 4], s[pos0 + 4] = 0.0, 1.0          # only token 4 turns
    out = oracle.rope_rows(x, c, s, pos0=pos0)
    keep = [t for t in range(6) if t != 4]
    np.testing.assert_array_equal(out[:, :, keep], x[:, :, keep])
    np.testing.assert_array_equal(out[:, :, 4, :2], -x[:, :, 4, 2:])


def test_rope_preserves_pair_norms_and_inverts():
    rng = np.random.default_rng(3)
    d, S = 16, 9
    x = rng.standard_normal((2, 1, S, d)).astype(np.float32)
    ang = rng.uniform(-np.pi, np.pi, (S, d // 2))
    c, s = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    y = oracle.rope_rows(x, c, s)
    n0 = x[..., :d // 2].astype(np.float64) ** 2 + x[..., d // 2:].astype(np.float64) ** 2
    n1 = y[..., :d // 2].astype(np.float64) ** 2 + y[..., d // 2:].astype(np.float64) ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-5, atol=1e-6)
    back = oracle.rope_rows(y, c, -s)
    np.testing.assert_allclose(back, x, rtol=1e-5, atol=1e-5)
    # a rotation by +a then +a is a rotation by 2a (angle addition), not the inverse
    twice = oracle.rope_rows(y, c, s)
    c2, s2 = np.cos(2 * ang).astype(np.float32), np.sin(2 * ang).astype(np.float32)
    np.testing.assert_allclose(twice, oracle.rope_rows(x, c2, s2), rtol=1e-4, atol=1e-5)


def test_calibration_hand_worked():
    q = np.zeros((1, 4, 3, 2))
    k = np.zeros((1, 2, 3, 2))
    q[0, 0, 1, 0], q[0, 1, 2, 0] = 0.5, -2.0     # group 0 (heads 0, 1): max |Q| = 2 on channel 0
    q[0, 3, 0, 0] = 8.0                          # group 1 only
    k[0, 0, :, 0] = [1.0, -8.0, 2.0]             # group 0: max |K| = 8
    k[0, 1, 2, 0] = 2.0                          # group 1: max |K| = 2
    q[0, 2, 0, 1], k[0, 1, 0, 1] = 1.0, 9.0      # group 1 channel 1: (9 / 1)^0.5 = 3
    s = oracle.smooth_calibrate(q, k, 0.5)
    assert s[0, 0] == 2.0                        # (8 / 2)^0.5
    assert s[1, 0] == 0.5                        # (2 / 8)^0.5
    assert s[0, 1] == 1.0                        # zero maxima give 1
    assert s[1, 1] == 3.0
    assert (oracle.smooth_calibrate(q, k, 0.0) == 1.0).all()   # x^0 = 1, and zero maxima give 1


@pytest.mark.parametrize("alpha", [0.5, 0.25, 1.0])
def test_calibration_balances_the_smoothed_maxima(alpha):
    rng = np.random.default_rng(4)
    q = rng.standard_normal((2, 4, 7, 8)) * rng.uniform(0.1, 5, 8)
    k = rng.standard_normal((2, 2, 7, 8)) * rng.uniform(0.1, 5, 8)
    s = oracle.smooth_calibrate(q, k, alpha).astype(np.float64)
    qm = np.abs(q).reshape(2, 2, 2, 7, 8).max(axis=(0, 2, 3))
    km = np.abs(k).max(axis=(0, 2))
    # max|Q s| and max|K / s|: equal at alpha = 1/2; the ratio moves by (km/qm)^(1-2 alpha)
    lhs = (km / s) / (qm * s)
    np.testing.assert_allclose(lhs, (km / qm) ** (1 - 2 * alpha), rtol=1e-6)
