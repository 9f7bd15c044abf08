"""hifa4_attn_fwd_noalloc, the entry point that allocates nothing (GPU).

Named to be collected last: it must pass after every other test of the run as well
as alone in a fresh process.

It runs the kernels of hifa4_attn_fwd with the decode partials in the
library's own device scratch instead of a caller workspace, so its outputs
must equal hifa4_attn_fwd's bit for bit.  Two decode calls in a row, the
second on a smaller batch, check that a call never depends on what the
previous one left in the shared scratch; a prefill call (no scratch) completes
it.  The refusal of a problem too large for the scratch is a host check
(tests/test_abi.py).
"""
import numpy as np
import pytest
import torch

from bit_flashattention_hifa4_amd import binding as hb
from bit_flashattention_hifa4_amd import workloads as W

pytestmark = pytest.mark.gpu


def _cache(cfg, lens, cap):
    B, Hq, Hkv, d = cfg.B, cfg.Hq, cfg.Hkv, cfg.d
    mx = hb.alloc_mx(B, Hq, Hkv, 1, cap, d)
    hb.hifa4_quantize_qkv(W.decode_q(cfg).cuda(), None, None, None, out=mx)
    for b, L in enumerate(lens):
        if int(L) == 0:
            continue
        k, v = W.decode_kv(cfg, b, int(L))
        sl = hb.MXQKV(None, None, mx.k_codes[b:b + 1], mx.k_scales[b:b + 1], mx.v_codes[b:b + 1],
                      mx.v_scales[b:b + 1], 1, Hq, Hkv, 0, int(L), d, cap)
        hb.hifa4_quantize_qkv(None, k.cuda(), v.cuda(), None, kv_stride=cap, out=sl)
    mx.Sq, mx.Sk, mx.kv_stride = 1, cap, cap
    return mx, torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()


def _both(mx, lens_t, chunk=0):
    kw = dict(causal=True, kv_lens=lens_t, decode_chunk=chunk,
              rescale_threshold=hb.RESCALE_THRESHOLD_FAST)
    o_ref, l_ref = hb.hifa4_attn_fwd(mx, **kw)
    out = torch.empty_like(o_ref)
    lse = torch.empty_like(l_ref)
    hb.hifa4_attn_fwd_noalloc(mx, out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    return (o_ref, l_ref), (out, lse)


@pytest.mark.parametrize("chunk", [0, 256])
def test_noalloc_decode_matches_workspace_entry_point_twice(chunk):
    big = W.DecodeConfig("noalloc_big", 16, 32, 8, 128, 5, 8192)
    lens_big = np.random.default_rng(5).integers(1, 8192, size=16)
    small = W.DecodeConfig("noalloc_small", 3, 8, 2, 128, 6, 700)
    lens_small = [700, 1, 333]
    for cfg, lens in ((big, lens_big), (small, lens_small)):
        print("noalloc decode:", cfg.name, "chunk", chunk, "sum(L)", int(np.sum(lens)), flush=True)
        cap = -(-int(max(lens)) // 64) * 64
        mx, lens_t = _cache(cfg, lens, cap)
        p = hb.make_params(cfg.B, cfg.Hq, cfg.Hkv, 1, cap, cfg.d, causal=True, kv_stride=cap,
                           kv_lens=lens_t, decode_chunk=chunk)
        assert 0 < hb.hifa4_attn_workspace_size(p) <= hb.NOALLOC_SCRATCH_BYTES
        (o_ref, l_ref), (o, l) = _both(mx, lens_t, chunk)
        assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
        assert torch.isfinite(o.float()).all()


def test_noalloc_prefill_matches_workspace_entry_point():
    inp = W.random_case(1, 4, 2, 200, 200, 128, dtype="bf16", seed=17, rope_theta=1e4,
                        n_outliers=2, smooth_alpha=0.5)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    s = torch.from_numpy(inp["smooth"]).cuda()
    mx = hb.hifa4_quantize_qkv(q, k, v, s)
    o_ref, l_ref = hb.hifa4_attn_fwd(mx, causal=True)
    out, lse = torch.empty_like(o_ref), torch.empty_like(l_ref)
    hb.hifa4_attn_fwd_noalloc(mx, causal=True, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out, o_ref) and torch.equal(lse, l_ref)
