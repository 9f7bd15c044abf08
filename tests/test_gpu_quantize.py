"""Smooth-QK + MXFP4 quantisation on the GPU vs the oracle: codes and scales bit-exact.

Covers the four prefill workloads at full size (tiny fp16 d64, Qwen3-8B-,
Llama-3.1-8B- and Gemma2-9B-shaped bf16), ragged token counts (tail value
blocks), a token capacity larger than Sk, GQA smoothing rows, fp16 input,
skipped tensors, and decode-cache construction into slices of a large cache.
"""
import numpy as np
import pytest
import torch

import oracle
from bit_flashattention_hifa4_amd import binding as hb
from bit_flashattention_hifa4_amd import workloads as W

pytestmark = pytest.mark.gpu


def _gpu_quantize(inp, kv_stride=0):
    q, k, v = (inp[n].cuda() if inp[n] is not None else None for n in ("q", "k", "v"))
    s = torch.from_numpy(inp["smooth"]).cuda() if inp["smooth"] is not None else None
    mx = hb.hifa4_quantize_qkv(q, k, v, s, kv_stride=kv_stride)
    torch.cuda.synchronize()
    return mx


def _check(inp, mx, kv_stride=0):
    f = lambda t: W.to_f32(t) if t is not None else None
    ref = oracle.quantize_qkv(f(inp["q"]), f(inp["k"]), f(inp["v"]), inp["smooth"],
                              kv_cap=kv_stride or None)
    Sk = inp["k"].shape[2] if inp["k"] is not None else 0
    if inp["q"] is not None:
        np.testing.assert_array_equal(mx.q_codes.cpu().numpy(), ref["q_codes"])
        np.testing.assert_array_equal(mx.q_scales.cpu().numpy(), ref["q_scales"])
    if inp["k"] is not None:
        np.testing.assert_array_equal(mx.k_codes.cpu().numpy()[:, :, :Sk], ref["k_codes"][:, :, :Sk])
        np.testing.assert_array_equal(mx.k_scales.cpu().numpy()[:, :, :Sk], ref["k_scales"][:, :, :Sk])
    if inp["v"] is not None:
        nb = (Sk + 31) // 32
        np.testing.assert_array_equal(mx.v_codes.cpu().numpy()[:, :, :nb], ref["v_codes"][:, :, :nb])
        np.testing.assert_array_equal(mx.v_scales.cpu().numpy()[:, :, :nb], ref["v_scales"][:, :, :nb])


@pytest.mark.parametrize("cfg", list(W.PREFILL_CONFIGS.values()), ids=lambda c: c.name)
def test_quantize_full_size_workloads_bit_exact(cfg):
    print("quantize parity:", cfg.name, flush=True)
    inp = W.prefill_inputs(cfg)
    mx = _gpu_quantize(inp)
    _check(inp, mx)


@pytest.mark.parametrize("case", [
    # B, Hq, Hkv, Sq, Sk, d, dtype, kv_stride, smooth
    (1, 2, 1, 37, 45, 64, "bf16", 0, True),
    (2, 4, 2, 5, 100, 128, "fp16", 160, True),
    (1, 8, 2, 1, 33, 256, "bf16", 64, False),
    (3, 3, 3, 64, 64, 128, "bf16", 0, True),
    (1, 1, 1, 1, 1, 64, "bf16", 0, True),
])
def test_quantize_ragged_and_strided(case):
    B, Hq, Hkv, Sq, Sk, d, dt, stride, sm = case
    print("quantize ragged:", case, flush=True)
    inp = W.random_case(B, Hq, Hkv, Sq, Sk, d, dtype=dt, seed=sum(case[:6]), n_outliers=2,
                        smooth_alpha=0.5 if sm else None, scale=3.0)
    mx = _gpu_quantize(inp, kv_stride=stride)
    _check(inp, mx, kv_stride=stride)


def test_quantize_extreme_values_bit_exact():
    """Values spanning the bf16 range, exact zeros, negative zeros and ties."""
    rng = np.random.default_rng(123)
    B, H, S, d = 1, 2, 96, 128
    x = (rng.standard_normal((B, H, S, d)) * np.exp2(rng.integers(-120, 120, size=(B, H, S, 1))))
    x[:, :, ::7] = 0.0
    x[:, :, 3::11, ::5] = -0.0
    x[:, :, 5, :] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 16) * 2.0 ** -3
    t = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    inp = dict(q=t, k=t.clone(), v=t.clone(), smooth=None)
    mx = _gpu_quantize(inp)
    _check(inp, mx)


def test_quantize_skips_tensors_and_builds_decode_cache_slices():
    cfg = W.DecodeConfig("small_decode", 4, 8, 2, 128, 40, 300)
    lens = [300, 41, 129, 64]
    cap = 320
    mx = hb.alloc_mx(cfg.B, cfg.Hq, cfg.Hkv, 1, cap, cfg.d)
    ks, vs = [], []
    for b, L in enumerate(lens):
        k, v = W.decode_kv(cfg, b, L)
        ks.append(k)
        vs.append(v)
        sl = hb.MXQKV(None, None, mx.k_codes[b:b + 1], mx.k_scales[b:b + 1], mx.v_codes[b:b + 1],
                      mx.v_scales[b:b + 1], 1, cfg.Hq, cfg.Hkv, 0, L, cfg.d, cap)
        hb.hifa4_quantize_qkv(None, k.cuda(), v.cuda(), None, kv_stride=cap, out=sl)
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        ref = oracle.quantize_qkv(None, W.to_f32(ks[b]), W.to_f32(vs[b]), None, kv_cap=cap)
        nb = (L + 31) // 32
        np.testing.assert_array_equal(mx.k_codes[b, :, :L].cpu().numpy(), ref["k_codes"][0, :, :L])
        np.testing.assert_array_equal(mx.k_scales[b, :, :L].cpu().numpy(), ref["k_scales"][0, :, :L])
        np.testing.assert_array_equal(mx.v_codes[b, :, :nb].cpu().numpy(), ref["v_codes"][0, :, :nb])
        np.testing.assert_array_equal(mx.v_scales[b, :, :nb].cpu().numpy(), ref["v_scales"][0, :, :nb])
