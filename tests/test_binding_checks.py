"""The Python binding refuses undersized or misshapen buffers (CPU only).

The C ABI receives bare device pointers and cannot know a buffer's size, so a
tensor smaller than what the kernels address would be written past its end on
the GPU.  The binding compares every buffer with the sizes of the documented
layouts (include/hifa4.h) and raises ValueError before anything is enqueued;
these tests use host tensors, which never reach a kernel.
"""
import pytest
import torch

from bit_flashattention_hifa4_amd import binding as hb

B, Hq, Hkv, S, d = 1, 4, 2, 64, 64


def _mx(cap=S, Sq=S):
    return hb.alloc_mx(B, Hq, Hkv, Sq, cap, d, device="cpu")


def _shrink(mx, name):
    t = getattr(mx, name)
    setattr(mx, name, t.reshape(-1)[:-1].clone())
    return mx


@pytest.mark.parametrize("name", ["q_codes", "q_scales", "k_codes", "k_scales", "v_codes",
                                  "v_scales"])
def test_attn_rejects_short_mx_buffer(name):
    mx = _shrink(_mx(), name)
    mx.Sq, mx.Sk = S, S
    out = torch.empty((B, Hq, S, d), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=name):
        hb.hifa4_attn_fwd(mx, causal=True, out=out, want_lse=False)


@pytest.mark.parametrize("shape,dtype,what", [
    ((B, Hq, S - 1, d), torch.bfloat16, "out"),
    ((B, Hq, S, d), torch.float32, "out"),
])
def test_attn_rejects_wrong_out(shape, dtype, what):
    mx = _mx()
    mx.Sq, mx.Sk = S, S
    with pytest.raises(ValueError, match=what):
        hb.hifa4_attn_fwd(mx, causal=True, out=torch.empty(shape, dtype=dtype), want_lse=False)


def test_attn_rejects_wrong_lse():
    mx = _mx()
    mx.Sq, mx.Sk = S, S
    out = torch.empty((B, Hq, S, d), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="lse"):
        hb.hifa4_attn_fwd(mx, causal=True, out=out, lse=torch.empty((B, Hq, S - 3)))


def test_qraw_rejects_short_kv_and_out():
    q = torch.empty((B, Hq, S, d), dtype=torch.bfloat16)
    mx = _shrink(_mx(), "v_scales")
    mx.Sk = S
    with pytest.raises(ValueError, match="v_scales"):
        hb.hifa4_attn_fwd_qraw(q, None, mx, causal=True, out=torch.empty_like(q),
                               want_lse=False)
    mx = _mx()
    mx.Sk = S
    with pytest.raises(ValueError, match="out"):
        hb.hifa4_attn_fwd_qraw(q, None, mx, causal=True, out=torch.empty((B, Hq, S, d - 1),
                                                                         dtype=q.dtype),
                               want_lse=False)


@pytest.mark.parametrize("name", ["q_codes", "k_scales", "v_codes"])
def test_quantize_rejects_short_output(name):
    q = torch.empty((B, Hq, S, d), dtype=torch.bfloat16)
    k = torch.empty((B, Hkv, S, d), dtype=torch.bfloat16)
    mx = _shrink(_mx(), name)
    with pytest.raises(ValueError, match=name):
        hb.hifa4_quantize_qkv(q, k, k.clone(), out=mx)


def test_quantize_rejects_capacity_beyond_the_buffers():
    k = torch.empty((B, Hkv, S, d), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="k_codes"):
        hb.hifa4_quantize_qkv(None, k, k.clone(), out=_mx(cap=S), kv_stride=2 * S)


def test_append_rejects_short_cache():
    k = torch.empty((B, Hkv, 1, d), dtype=torch.bfloat16)
    lens = torch.zeros(B, dtype=torch.int32)
    cache = _shrink(_mx(cap=128, Sq=1), "k_codes")
    tail = torch.zeros((B, Hkv, 32, d), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="k_codes"):
        hb.hifa4_kv_append(None, k, k.clone(), lens, cache, tail)


def test_bf16_rejects_wrong_out_and_kv():
    q = torch.empty((B, Hq, S, d), dtype=torch.bfloat16)
    k = torch.empty((B, Hkv, S, d), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out"):
        hb.bf16_attn_fwd(q, k, k.clone(), causal=True, out=torch.empty((B, Hq, S, 2 * d),
                                                                      dtype=q.dtype))
    with pytest.raises(ValueError, match="k and v"):
        hb.bf16_attn_fwd(q, k, k[:, :, :S - 1].clone(), causal=True)
