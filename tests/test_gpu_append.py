"""MXFP4 KV-cache append on the GPU vs the oracle.

The append's result has a plain definition: after any sequence of appends the
cache holds what the oracle's one-shot RoPE + Smooth-QK + MXFP4 quantisation
of each whole sequence gives (token t rotated at position t), and the new
queries are the oracle's quantisation of the rotated queries at positions
L_b + i.  Checked bit for bit with per-sequence lengths that start mid-block,
appends of 1 token and of many (crossing several value blocks), a cache
built in bulk first (tail filled by the caller), the decode step end to end
(append then attention, identical to attention over a one-shot cache), the
capacity clamp, n = 0, and one append into the full-size decode cache
(B64 Hq32 Hkv8 d128, capacity 32768, lengths 1k-32k).
"""
import numpy as np
import pytest
import torch

import oracle
from bit_flashattention_hifa4_amd import binding as hb
from bit_flashattention_hifa4_amd import workloads as W

pytestmark = pytest.mark.gpu


def _draw(rng, shape, dt):
    x = rng.standard_normal(shape, dtype=np.float32) * np.float32(2.0)
    return torch.from_numpy(x).to(dt)


def _oracle_cache(kseq, vseq, smooth, cos, sin, cap, rule=0):
    """One-shot oracle quantisation of one sequence's K, V [1, Hkv, L, d] (torch)."""
    k = oracle.rope_rows(W.to_f32(kseq), cos, sin, 0) if cos is not None else W.to_f32(kseq)
    return oracle.quantize_qkv(None, k, W.to_f32(vseq), smooth, kv_cap=cap, rule=rule)


def _check_seq(cache, b, L, ref):
    nb = (L + 31) // 32
    np.testing.assert_array_equal(cache.k_codes[b, :, :L].cpu().numpy(), ref["k_codes"][0, :, :L])
    np.testing.assert_array_equal(cache.k_scales[b, :, :L].cpu().numpy(), ref["k_scales"][0, :, :L])
    np.testing.assert_array_equal(cache.v_codes[b, :, :nb].cpu().numpy(), ref["v_codes"][0, :, :nb])
    np.testing.assert_array_equal(cache.v_scales[b, :, :nb].cpu().numpy(), ref["v_scales"][0, :, :nb])


@pytest.mark.parametrize("case", [
    # B, Hq, Hkv, d, dtype, cap, start lengths, appends, rope theta or None, smooth
    (3, 8, 2, 128, "bf16", 200, (0, 7, 33), (5, 1, 1, 30, 27, 64, 1, 3), 1e6, True),
    (2, 4, 4, 64, "fp16", 130, (31, 64), (1, 1, 2, 33, 1), 1e4, False),
    (2, 16, 8, 256, "bf16", 96, (32, 0), (40, 1, 23), None, True),
])
@pytest.mark.parametrize("rule", [hb.SCALE_OCP, hb.SCALE_NOCLIP])
def test_appends_equal_one_shot_quantisation(case, rule):
    """Under either block-scale rule (the cache's), appends equal a one-shot quantisation."""
    B, Hq, Hkv, d, dt, cap, starts, steps, theta, sm = case
    print("kv append:", case, "scale rule", rule, flush=True)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float16
    rng = np.random.default_rng(sum(starts) + cap)
    smooth = np.exp2(rng.uniform(-1, 1, (Hkv, d))).astype(np.float32) if sm else None
    smooth_t = torch.from_numpy(smooth).cuda() if sm else None
    cos = sin = cos_t = sin_t = None
    if theta is not None:
        cos, sin = W.rope_tables(cap + 8, d, theta)
        cos_t, sin_t = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    cache = hb.alloc_mx(B, Hq, Hkv, 1, cap, d, scale_rule=rule)
    tail = hb.alloc_v_tail(B, Hkv, d, dtype=tdt)
    # sequence b starts with starts[b] tokens quantised in bulk; the caller fills the tail
    kseq = [_draw(rng, (1, Hkv, L, d), tdt) for L in starts]
    vseq = [_draw(rng, (1, Hkv, L, d), tdt) for L in starts]
    for b, L in enumerate(starts):
        if L == 0:
            continue
        sl = hb.MXQKV(None, None, cache.k_codes[b:b + 1], cache.k_scales[b:b + 1],
                      cache.v_codes[b:b + 1], cache.v_scales[b:b + 1], 1, Hq, Hkv, 0, L, d, cap)
        if theta is not None:
            hb.hifa4_quantize_qkv_rope(None, kseq[b].cuda(), vseq[b].cuda(), cos_t, sin_t,
                                       smooth=smooth_t, kv_stride=cap, out=sl, Hkv=Hkv,
                                       scale_rule=rule)
        else:
            hb.hifa4_quantize_qkv(None, kseq[b].cuda(), vseq[b].cuda(), smooth_t, kv_stride=cap,
                                  out=sl, scale_rule=rule)
        r = L % 32
        if r:
            tail[b, :, :r] = vseq[b][0, :, L - r:].cuda()
    lens = torch.tensor(starts, dtype=torch.int32, device="cuda")
    for step, n in enumerate(steps):
        q = _draw(rng, (B, Hq, n, d), tdt)
        k = _draw(rng, (B, Hkv, n, d), tdt)
        v = _draw(rng, (B, Hkv, n, d), tdt)
        qc = hb.alloc_mx(B, Hq, Hkv, n, cap, d)
        step_cache = hb.MXQKV(qc.q_codes, qc.q_scales, cache.k_codes, cache.k_scales,
                              cache.v_codes, cache.v_scales, B, Hq, Hkv, n, cap, d, cap, rule)
        lens_out = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        hb.hifa4_kv_append(q.cuda(), k.cuda(), v.cuda(), lens, step_cache, tail,
                           kv_lens_out=lens_out, smooth=smooth_t, cos=cos_t, sin=sin_t)
        torch.cuda.synchronize()
        L = lens.cpu().numpy()
        np.testing.assert_array_equal(lens_out.cpu().numpy(), L + n)
        for b in range(B):
            qf = W.to_f32(q[b:b + 1])
            if theta is not None:
                qf = oracle.rope_rows(qf, cos, sin, int(L[b]))
            ref_q = oracle.quantize_rows(qf, smooth, divide=False, rule=rule)
            np.testing.assert_array_equal(qc.q_codes[b:b + 1].cpu().numpy(), ref_q[0])
            np.testing.assert_array_equal(qc.q_scales[b:b + 1].cpu().numpy(), ref_q[1])
            kseq[b] = torch.cat([kseq[b], k[b:b + 1]], dim=2)
            vseq[b] = torch.cat([vseq[b], v[b:b + 1]], dim=2)
        lens = lens_out
    for b in range(B):
        Lb = kseq[b].shape[2]
        _check_seq(cache, b, Lb, _oracle_cache(kseq[b], vseq[b], smooth, cos, sin, cap, rule))
        r = Lb % 32
        if r:   # the tail holds the raw values of the open block
            assert torch.equal(tail[b, :, :r].cpu(), vseq[b][0, :, Lb - r:])


def test_decode_step_append_then_attention_matches_one_shot_cache():
    B, Hq, Hkv, d, cap = 4, 16, 4, 128, 320
    starts = [100, 31, 32, 257]
    rng = np.random.default_rng(9)
    tdt = torch.bfloat16
    cos, sin = W.rope_tables(cap, d, 1e6)
    cos_t, sin_t = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    kseq = [_draw(rng, (1, Hkv, L, d), tdt) for L in starts]
    vseq = [_draw(rng, (1, Hkv, L, d), tdt) for L in starts]
    qn = _draw(rng, (B, Hq, 1, d), tdt)
    kn = _draw(rng, (B, Hkv, 1, d), tdt)
    vn = _draw(rng, (B, Hkv, 1, d), tdt)
    # path 1: bulk cache of the first L_b tokens, then the decode-step append
    cache = hb.alloc_mx(B, Hq, Hkv, 1, cap, d)
    tail = hb.alloc_v_tail(B, Hkv, d)
    for b, L in enumerate(starts):
        sl = hb.MXQKV(None, None, cache.k_codes[b:b + 1], cache.k_scales[b:b + 1],
                      cache.v_codes[b:b + 1], cache.v_scales[b:b + 1], 1, Hq, Hkv, 0, L, d, cap)
        hb.hifa4_quantize_qkv_rope(None, kseq[b].cuda(), vseq[b].cuda(), cos_t, sin_t,
                                   kv_stride=cap, out=sl, Hkv=Hkv)
        if L % 32:
            tail[b, :, :L % 32] = vseq[b][0, :, L - L % 32:].cuda()
    lens = torch.tensor(starts, dtype=torch.int32, device="cuda")
    lens_new = torch.empty_like(lens)
    hb.hifa4_kv_append(qn.cuda(), kn.cuda(), vn.cuda(), lens, cache, tail, kv_lens_out=lens_new,
                       cos=cos_t, sin=sin_t)
    o1, l1 = hb.hifa4_attn_fwd(cache, causal=True, kv_lens=lens_new)
    # path 2: one-shot cache of the L_b + 1 tokens, query quantised at its position
    ref = hb.alloc_mx(B, Hq, Hkv, 1, cap, d)
    for b, L in enumerate(starts):
        kk = torch.cat([kseq[b], kn[b:b + 1]], dim=2).cuda()
        vv = torch.cat([vseq[b], vn[b:b + 1]], dim=2).cuda()
        sl = hb.MXQKV(ref.q_codes[b:b + 1], ref.q_scales[b:b + 1], ref.k_codes[b:b + 1],
                      ref.k_scales[b:b + 1], ref.v_codes[b:b + 1], ref.v_scales[b:b + 1], 1, Hq,
                      Hkv, 1, L + 1, d, cap)
        hb.hifa4_quantize_qkv_rope(qn[b:b + 1].cuda(), kk, vv, cos_t, sin_t, q_pos0=L,
                                   kv_stride=cap, out=sl)
    ref.Sq, ref.Sk = 1, cap
    o2, l2 = hb.hifa4_attn_fwd(ref, causal=True, kv_lens=lens_new)
    torch.cuda.synchronize()
    assert lens_new.cpu().tolist() == [L + 1 for L in starts]
    assert torch.equal(cache.q_codes, ref.q_codes) and torch.equal(cache.q_scales, ref.q_scales)
    for b, L in enumerate(starts):
        nb = (L + 1 + 31) // 32
        assert torch.equal(cache.k_codes[b, :, :L + 1], ref.k_codes[b, :, :L + 1])
        assert torch.equal(cache.k_scales[b, :, :L + 1], ref.k_scales[b, :, :L + 1])
        assert torch.equal(cache.v_codes[b, :, :nb], ref.v_codes[b, :, :nb])
        assert torch.equal(cache.v_scales[b, :, :nb], ref.v_scales[b, :, :nb])
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_append_clamps_at_capacity_and_handles_empty_appends():
    B, Hq, Hkv, d, cap = 3, 4, 2, 64, 70
    rng = np.random.default_rng(4)
    cache = hb.alloc_mx(B, Hq, Hkv, 1, cap, d)
    for t in (cache.k_codes, cache.k_scales, cache.v_codes, cache.v_scales):
        t.fill_(0xAB)
    tail = hb.alloc_v_tail(B, Hkv, d)
    k = _draw(rng, (B, Hkv, 5, d), torch.bfloat16).cuda()
    v = _draw(rng, (B, Hkv, 5, d), torch.bfloat16).cuda()
    # sequence 0 would overflow (68 + 5 > 70); sequence 1's length is negative (-> 0)
    lens = torch.tensor([68, -3, 10], dtype=torch.int32, device="cuda")
    out = torch.empty_like(lens)
    before_k = cache.k_codes.clone()
    hb.hifa4_kv_append(None, k, v, lens, cache, tail, kv_lens_out=out)
    torch.cuda.synchronize()
    assert out.cpu().tolist() == [70, 5, 15]
    # rows written: seq 0 rows 68, 69; seq 1 rows 0..4; seq 2 rows 10..14 -- nothing else
    changed = (cache.k_codes != before_k).any(dim=-1).cpu().numpy()   # [B, Hkv, cap]
    expect = np.zeros_like(changed)
    expect[0, :, 68:70] = True
    expect[1, :, 0:5] = True
    expect[2, :, 10:15] = True
    assert not np.any(changed & ~expect)
    # n = 0: lengths pass through, nothing is written
    snap = [t.clone() for t in (cache.k_codes, cache.v_codes, tail)]
    e = torch.empty((B, Hkv, 0, d), dtype=torch.bfloat16, device="cuda")
    hb.hifa4_kv_append(None, e, e, out, cache, tail, kv_lens_out=lens)
    torch.cuda.synchronize()
    assert lens.cpu().tolist() == [70, 5, 15]
    for a, b in zip(snap, (cache.k_codes, cache.v_codes, tail)):
        assert torch.equal(a, b)


def test_append_into_full_size_decode_cache():
    cfg = W.DECODE
    B, Hq, Hkv, d, cap = cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.max_len
    print("kv append full size:", cfg.name, flush=True)
    L = W.decode_lengths(cfg)
    assert L.max() < cap
    rng = np.random.default_rng(cfg.seed + 77)
    cache = hb.alloc_mx(B, Hq, Hkv, 1, cap, d)
    for t in (cache.k_codes, cache.k_scales, cache.v_codes, cache.v_scales):
        t.fill_(0x5C)
    tail_h = _draw(rng, (B, Hkv, 32, d), torch.bfloat16)
    tail = tail_h.cuda()
    cos, sin = W.rope_tables(cap + 1, d, 1e6)
    qn = _draw(rng, (B, Hq, 1, d), torch.bfloat16)
    kn = _draw(rng, (B, Hkv, 1, d), torch.bfloat16)
    vn = _draw(rng, (B, Hkv, 1, d), torch.bfloat16)
    lens = torch.from_numpy(L).cuda()
    lens_new = torch.empty_like(lens)
    hb.hifa4_kv_append(qn.cuda(), kn.cuda(), vn.cuda(), lens, cache, tail, kv_lens_out=lens_new,
                       cos=torch.from_numpy(cos).cuda(), sin=torch.from_numpy(sin).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(lens_new.cpu().numpy(), L + 1)
    kc, ks = cache.k_codes.cpu().numpy(), cache.k_scales.cpu().numpy()
    vc, vs = cache.v_codes.cpu().numpy(), cache.v_scales.cpu().numpy()
    qc, qs = cache.q_codes.cpu().numpy(), cache.q_scales.cpu().numpy()
    for b in range(B):
        Lb = int(L[b])
        rq = oracle.quantize_rows(oracle.rope_rows(W.to_f32(qn[b:b + 1]), cos, sin, Lb), None,
                                  divide=False)
        np.testing.assert_array_equal(qc[b:b + 1], rq[0])
        np.testing.assert_array_equal(qs[b:b + 1], rq[1])
        rk = oracle.quantize_rows(oracle.rope_rows(W.to_f32(kn[b:b + 1]), cos, sin, Lb), None,
                                  divide=True)
        np.testing.assert_array_equal(kc[b:b + 1, :, Lb], rk[0][:, :, 0])
        np.testing.assert_array_equal(ks[b:b + 1, :, Lb], rk[1][:, :, 0])
        r = Lb % 32
        blk = torch.cat([tail_h[b:b + 1, :, :r], vn[b:b + 1]], dim=2)
        rv = oracle.quantize_v(W.to_f32(blk))
        np.testing.assert_array_equal(vc[b, :, Lb // 32], rv[0][0, :, 0])
        np.testing.assert_array_equal(vs[b, :, Lb // 32], rv[1][0, :, 0])
        if r != 31:   # the block stays open: its new token's raw value is in the tail
            assert torch.equal(tail[b, :, r].cpu(), vn[b, :, 0])
    # nothing else changed
    touched_k = np.zeros((B, Hkv, cap), bool)
    touched_v = np.zeros((B, Hkv, (cap + 31) // 32), bool)
    for b in range(B):
        touched_k[b, :, L[b]] = True
        touched_v[b, :, L[b] // 32] = True
    assert np.all(kc[~touched_k] == 0x5C) and np.all(ks[~touched_k] == 0x5C)
    assert np.all(vc[~touched_v] == 0x5C) and np.all(vs[~touched_v] == 0x5C)
