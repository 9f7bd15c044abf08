"""RoPE inside the quantiser and the Smooth-QK calibration on the GPU vs the oracle.

RoPE + Smooth-QK + MXFP4: codes and scales bit-exact against the oracle's
rotation (fp32 products, no contraction) followed by its quantiser, over head
dims 64 / 128 / 256, bf16 and fp16, ragged token counts, nonzero start
positions (decode: one token at position L - 1), a token capacity above Sk,
GQA smoothing rows and one Qwen3-8B-shaped full-size case.  Calibration:
within one fp32 ulp of the oracle (the fp64 power is the device's pow), with
and without the rotation, across the 256-token chunk boundary, with all-zero
channels (s = 1) and an empty calibration set.
"""
import numpy as np
import pytest
import torch

import oracle
from bit_flashattention_hifa4_amd import binding as hb
from bit_flashattention_hifa4_amd import workloads as W

pytestmark = pytest.mark.gpu


def _oracle_codes(inp, cos, sin, q_pos0, k_pos0, kv_stride):
    f = lambda t: W.to_f32(t) if t is not None else None
    q = oracle.rope_rows(f(inp["q"]), cos, sin, q_pos0) if inp["q"] is not None else None
    k = oracle.rope_rows(f(inp["k"]), cos, sin, k_pos0) if inp["k"] is not None else None
    return oracle.quantize_qkv(q, k, f(inp["v"]), inp["smooth"], kv_cap=kv_stride or None)


def _check_codes(inp, mx, ref):
    Sk = inp["k"].shape[2]
    nb = (Sk + 31) // 32
    np.testing.assert_array_equal(mx.q_codes.cpu().numpy(), ref["q_codes"])
    np.testing.assert_array_equal(mx.q_scales.cpu().numpy(), ref["q_scales"])
    np.testing.assert_array_equal(mx.k_codes.cpu().numpy()[:, :, :Sk], ref["k_codes"][:, :, :Sk])
    np.testing.assert_array_equal(mx.k_scales.cpu().numpy()[:, :, :Sk], ref["k_scales"][:, :, :Sk])
    np.testing.assert_array_equal(mx.v_codes.cpu().numpy()[:, :, :nb], ref["v_codes"][:, :, :nb])
    np.testing.assert_array_equal(mx.v_scales.cpu().numpy()[:, :, :nb], ref["v_scales"][:, :, :nb])


def _run_rope(inp, cos, sin, q_pos0, k_pos0, kv_stride=0):
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    s = torch.from_numpy(inp["smooth"]).cuda() if inp["smooth"] is not None else None
    mx = hb.hifa4_quantize_qkv_rope(q, k, v, torch.from_numpy(cos).cuda(),
                                    torch.from_numpy(sin).cuda(), q_pos0=q_pos0, k_pos0=k_pos0,
                                    smooth=s, kv_stride=kv_stride)
    torch.cuda.synchronize()
    return mx


@pytest.mark.parametrize("case", [
    # B, Hq, Hkv, Sq, Sk, d, dtype, kv_stride, smooth, q_pos0, k_pos0, theta
    (1, 2, 1, 37, 45, 64, "bf16", 0, True, 8, 0, 1e4),
    (2, 4, 2, 100, 100, 128, "fp16", 160, True, 0, 0, 1e6),
    (1, 8, 2, 33, 33, 256, "bf16", 64, False, 3, 3, 1e4),
    (3, 3, 3, 64, 64, 128, "bf16", 0, True, 500, 500, 5e5),
    (2, 8, 2, 1, 1, 128, "bf16", 0, True, 1023, 1023, 1e6),   # decode: one new token
    (1, 4, 4, 129, 200, 64, "fp16", 0, True, 71, 0, 1e4),
])
def test_rope_quantize_bit_exact(case):
    B, Hq, Hkv, Sq, Sk, d, dt, stride, sm, qp, kp, theta = case
    print("rope quantize:", case, flush=True)
    inp = W.random_case(B, Hq, Hkv, Sq, Sk, d, dtype=dt, seed=7 + sum(case[:6]), n_outliers=2,
                        smooth_alpha=0.5 if sm else None, scale=3.0)
    cos, sin = W.rope_tables(max(qp + Sq, kp + Sk) + 5, d, theta)
    mx = _run_rope(inp, cos, sin, qp, kp, stride)
    _check_codes(inp, mx, _oracle_codes(inp, cos, sin, qp, kp, stride))


def test_rope_quantize_full_size_qwen3_bit_exact():
    cfg = W.QWEN3_8B
    print("rope quantize full size:", cfg.name, flush=True)
    inp = W.prefill_inputs(cfg)   # treated as pre-rotation activations
    cos, sin = W.rope_tables(cfg.S, cfg.d, 1e6)
    mx = _run_rope(inp, cos, sin, 0, 0)
    _check_codes(inp, mx, _oracle_codes(inp, cos, sin, 0, 0, 0))


def test_rope_identity_tables_match_plain_quantize():
    """cos = 1, sin = 0 is no rotation: the codes equal hifa4_quantize_qkv's."""
    inp = W.random_case(2, 4, 2, 70, 70, 128, seed=3, smooth_alpha=0.5)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    s = torch.from_numpy(inp["smooth"]).cuda()
    ones = torch.ones((70, 64), dtype=torch.float32, device="cuda")
    a = hb.hifa4_quantize_qkv_rope(q, k, v, ones, torch.zeros_like(ones), smooth=s)
    b = hb.hifa4_quantize_qkv(q, k, v, s)
    torch.cuda.synchronize()
    for n in ("q_codes", "q_scales", "k_codes", "k_scales", "v_codes", "v_scales"):
        assert torch.equal(getattr(a, n), getattr(b, n)), n


def _ulps(a, b):
    return np.abs(a.view(np.int32).astype(np.int64) - b.view(np.int32).astype(np.int64))


def _calib_case(B, Hq, Hkv, S, d, dt, seed, zero_channels=False):
    inp = W.random_case(B, Hq, Hkv, S, S, d, dtype=dt, seed=seed, n_outliers=3, scale=2.0)
    q, k = inp["q"], inp["k"]
    if zero_channels:
        q[:, :, :, 5] = 0     # every query head: s = 1 on channel 5
        k[:, 0, :, 9] = 0     # kv head 0: s = 1 on channel 9
    return q, k


@pytest.mark.parametrize("case", [
    # B, Hq, Hkv, S, d, dtype, alpha, rope (q_pos0, k_pos0) or None
    (1, 4, 1, 300, 128, "bf16", 0.5, None),
    (2, 8, 2, 257, 64, "fp16", 0.25, None),
    (1, 16, 8, 512, 256, "bf16", 0.75, None),
    (3, 6, 3, 45, 128, "bf16", 0.5, (0, 0)),
    (1, 4, 2, 600, 64, "fp16", 1.0, (17, 40)),
    (2, 2, 2, 1, 128, "bf16", 0.5, (9, 9)),
])
def test_calibrate_matches_oracle(case):
    B, Hq, Hkv, S, d, dt, alpha, rope = case
    print("calibrate:", case, flush=True)
    q, k = _calib_case(B, Hq, Hkv, S, d, dt, seed=11 + S, zero_channels=True)
    qf, kf = W.to_f32(q), W.to_f32(k)
    kw = {}
    if rope is not None:
        cos, sin = W.rope_tables(max(rope) + S + 3, d, 1e4)
        qf = oracle.rope_rows(qf, cos, sin, rope[0])
        kf = oracle.rope_rows(kf, cos, sin, rope[1])
        kw = dict(cos=torch.from_numpy(cos).cuda(), sin=torch.from_numpy(sin).cuda(),
                  q_pos0=rope[0], k_pos0=rope[1])
    ref = oracle.smooth_calibrate(qf, kf, alpha)
    got = hb.hifa4_smooth_calibrate(q.cuda(), k.cuda(), alpha, **kw).cpu().numpy()
    assert got.shape == ref.shape
    assert _ulps(got, ref).max() <= 1, (got, ref)
    if rope is None:   # a rotation mixes the zeroed channel with its partner
        assert np.all(got[:, 5] == 1.0) and got[0, 9] == 1.0


def test_calibrate_reuses_workspace_and_empty_set_gives_ones():
    q, k = _calib_case(1, 4, 2, 40, 128, "bf16", seed=5)
    ws = torch.full((hb.hifa4_smooth_calibrate_workspace_size(2, 128),), 0xFF, dtype=torch.uint8,
                    device="cuda")   # stale contents must not leak into the maxima
    a = hb.hifa4_smooth_calibrate(q.cuda(), k.cuda(), 0.5, workspace=ws).cpu().numpy()
    ref = oracle.smooth_calibrate(W.to_f32(q), W.to_f32(k), 0.5)
    assert _ulps(a, ref).max() <= 1
    e = torch.empty((1, 4, 0, 128), dtype=torch.bfloat16, device="cuda")
    ones = hb.hifa4_smooth_calibrate(e, e[:, :2], 0.5, workspace=ws).cpu().numpy()
    np.testing.assert_array_equal(ones, np.ones((2, 128), np.float32))


def test_calibrate_full_calibration_set_qwen3():
    cfg = W.QWEN3_8B
    print("calibrate full set:", cfg.name, flush=True)
    q, k, _ = W._draw_qkv(cfg, cfg.seed + 1, 1, 4096)
    got = hb.hifa4_smooth_calibrate(q.cuda(), k.cuda(), cfg.smooth_alpha).cpu().numpy()
    ref = oracle.smooth_calibrate(W.to_f32(q), W.to_f32(k), cfg.smooth_alpha)
    assert _ulps(got, ref).max() <= 1
