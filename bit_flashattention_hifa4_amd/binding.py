"""ctypes binding of libhifa4.so (C ABI: include/hifa4.h).

Argument marshalling only: every step of the attention path runs in the HIP
kernels behind these calls.  PyTorch supplies device memory (the caller's
tensors, or ``torch.empty`` for outputs the caller did not pass) and the
current HIP stream.  There is no CPU fallback: if the library is missing or
the tensors are not on the GPU, the calls raise.

The Python names match the C entry points: ``hifa4_quantize_qkv``,
``hifa4_quantize_qkv_rope``, ``hifa4_kv_append``, ``hifa4_smooth_calibrate``,
``hifa4_smooth_calibrate_workspace_size``, ``hifa4_attn_fwd``, ``hifa4_attn_fwd_noalloc``,
``hifa4_attn_fwd_qraw``, ``bf16_attn_fwd``, ``hifa4_attn_schedule``,
``hifa4_attn_decode_piece_tiles``, ``hifa4_attn_workspace_size``,
``hifa4_status_string``, ``hifa4_last_error``.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhifa4.so")

HIFA4_OK = 0
HIFA4_ERR_INVALID_ARGUMENT = -1
HIFA4_ERR_UNSUPPORTED = -2
HIFA4_ERR_WORKSPACE_TOO_SMALL = -3
HIFA4_ERR_HIP = -4
HIFA4_BF16 = 0
HIFA4_FP16 = 1
SCALE_OCP = 0     # hifa4_scale_rule: OCP MX shared exponent
SCALE_NOCLIP = 1  # one higher wherever OCP would saturate an element

# Device scratch behind hifa4_attn_fwd_noalloc, per GPU (HIFA4_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 16 << 20

# Lazy-rescale threshold (log2 units) the benchmark and the full-size tests run
# with: a row's running max moves only when a key tile raises it by more than
# 2^8, which removes nearly every accumulator rescale.  0 is the
# FlashAttention-2 frame.  Exact attention is the same for both; P_hat is not,
# and the CPU oracle takes the same value.
RESCALE_THRESHOLD_FAST = 8.0


class HiFA4Error(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__("%s (%d): %s" % (hifa4_status_string(status), status, detail))
        self.status = status


class MxTensorC(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("scale_rule", ctypes.c_int32)]


class AttnParamsC(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Sq", ctypes.c_int32), ("Sk", ctypes.c_int32), ("d", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("sm_scale", ctypes.c_float),
        ("kv_stride", ctypes.c_int32), ("kv_lens", ctypes.c_void_p),
        ("decode_chunk", ctypes.c_int32), ("rescale_threshold", ctypes.c_float),
        ("normaliser", ctypes.c_int32),
        ("scale_rule", ctypes.c_int32),
    ]

class RopeC(ctypes.Structure):
    _fields_ = [("cos", ctypes.c_void_p), ("sin", ctypes.c_void_p), ("n_pos", ctypes.c_int32),
                ("q_pos0", ctypes.c_int32), ("k_pos0", ctypes.c_int32)]


NORMALISER_P_REORDERING = 0   # l = sum(P_hat) through the ones column (the method)
NORMALISER_DIRECT = 1         # l = sum(P) in fp32 on the vector ALU (the pages' comparison)


_lib = None


def load_library(path: str = LIB_PATH):
    """Open libhifa4.so; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            "libhifa4.so is not built (%s). Build it with `python -m "
            "bit_flashattention_hifa4_amd.build`; there is no CPU fallback." % path)
    lib = ctypes.CDLL(path)
    st = ctypes.c_int
    vp = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.hifa4_quantize_qkv.restype = st
    lib.hifa4_quantize_qkv.argtypes = [vp, vp, vp, st, i32, i32, i32, i32, i32, i32, i32, vp,
                                       MxTensorC, MxTensorC, MxTensorC, vp]
    lib.hifa4_quantize_qkv_rope.restype = st
    lib.hifa4_quantize_qkv_rope.argtypes = [vp, vp, vp, st, i32, i32, i32, i32, i32, i32, i32, vp,
                                            ctypes.POINTER(RopeC), MxTensorC, MxTensorC,
                                            MxTensorC, vp]
    lib.hifa4_kv_append.restype = st
    lib.hifa4_kv_append.argtypes = [vp, vp, vp, st, i32, i32, i32, i32, i32, i32, vp, vp, vp,
                                    ctypes.POINTER(RopeC), vp, MxTensorC, MxTensorC, MxTensorC,
                                    vp]
    lib.hifa4_smooth_calibrate_workspace_size.restype = ctypes.c_size_t
    lib.hifa4_smooth_calibrate_workspace_size.argtypes = [i32, i32]
    lib.hifa4_smooth_calibrate.restype = st
    lib.hifa4_smooth_calibrate.argtypes = [vp, vp, st, i32, i32, i32, i32, i32,
                                           ctypes.POINTER(RopeC), ctypes.c_double, vp, vp,
                                           ctypes.c_size_t, vp]
    lib.hifa4_attn_workspace_size.restype = ctypes.c_size_t
    lib.hifa4_attn_workspace_size.argtypes = [ctypes.POINTER(AttnParamsC)]
    lib.hifa4_attn_fwd.restype = st
    lib.hifa4_attn_fwd.argtypes = [ctypes.POINTER(AttnParamsC), MxTensorC, MxTensorC, MxTensorC,
                                   vp, st, vp, vp, ctypes.c_size_t, vp]
    lib.hifa4_attn_fwd_noalloc.restype = st
    lib.hifa4_attn_fwd_noalloc.argtypes = [ctypes.POINTER(AttnParamsC), MxTensorC, MxTensorC,
                                           MxTensorC, vp, st, vp, vp]
    lib.hifa4_attn_fwd_qraw.restype = st
    lib.hifa4_attn_fwd_qraw.argtypes = [ctypes.POINTER(AttnParamsC), vp, st, vp, MxTensorC,
                                        MxTensorC, vp, st, vp, vp, ctypes.c_size_t, vp]
    lib.bf16_attn_fwd.restype = st
    lib.bf16_attn_fwd.argtypes = [ctypes.POINTER(AttnParamsC), vp, vp, vp, vp, vp, vp,
                                  ctypes.c_size_t, vp]
    lib.hifa4_attn_schedule.restype = st
    lib.hifa4_attn_schedule.argtypes = [ctypes.POINTER(AttnParamsC), ctypes.POINTER(i32),
                                        ctypes.POINTER(i32)]
    lib.hifa4_attn_decode_piece_tiles.restype = i32
    lib.hifa4_attn_decode_piece_tiles.argtypes = [ctypes.POINTER(AttnParamsC), ctypes.c_int64]
    lib.hifa4_status_string.restype = ctypes.c_char_p
    lib.hifa4_status_string.argtypes = [st]
    lib.hifa4_last_error.restype = ctypes.c_char_p
    lib.hifa4_last_error.argtypes = []
    _lib = lib
    return lib


def hifa4_status_string(status: int) -> str:
    return load_library().hifa4_status_string(int(status)).decode()


def hifa4_last_error() -> str:
    return load_library().hifa4_last_error().decode()


def _check(status: int) -> None:
    if status != HIFA4_OK:
        raise HiFA4Error(status, hifa4_last_error())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU (the library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return HIFA4_BF16
    if dt == torch.float16:
        return HIFA4_FP16
    raise ValueError("dtype must be bfloat16 or float16, got %s" % dt)


def _need_bytes(t: Optional[torch.Tensor], nbytes: int, name: str) -> None:
    """The C ABI takes bare pointers and cannot see sizes: a buffer smaller than what the
    kernels address is refused here, before anything is enqueued."""
    if t is None:
        raise ValueError("%s is missing" % name)
    if t.dtype != torch.uint8:
        raise ValueError("%s must be uint8, got %s" % (name, t.dtype))
    if t.numel() < nbytes:
        raise ValueError("%s holds %d bytes, the call addresses %d" % (name, t.numel(), nbytes))


def _need_shape(t: torch.Tensor, shape, dtypes, name: str) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.dtype not in dtypes:
        raise ValueError("%s has dtype %s (allowed: %s)" % (name, t.dtype, dtypes))


def _check_row_mx(codes, scales, rows: int, d: int, name: str) -> None:
    """Row layout (queries, keys): rows x d/2 code bytes and rows x d/32 scale bytes."""
    _need_bytes(codes, rows * (d // 2), name + "_codes")
    _need_bytes(scales, rows * (d // 32), name + "_scales")


def _check_col_mx(codes, scales, heads: int, cap: int, d: int, name: str) -> None:
    """Column layout (values): ceil(cap / 32) blocks of d x 16 code bytes and d scales."""
    nblk = (cap + 31) // 32
    _need_bytes(codes, heads * nblk * d * 16, name + "_codes")
    _need_bytes(scales, heads * nblk * d, name + "_scales")


def _check_out_lse(out, lse, B, Hq, Sq, d) -> None:
    _need_shape(out, (B, Hq, Sq, d), (torch.bfloat16, torch.float16), "out")
    if lse is not None:
        _need_shape(lse, (B, Hq, Sq), (torch.float32,), "lse")


@dataclasses.dataclass
class MXQKV:
    """Quantised operands in the library's layouts (see include/hifa4.h)."""
    q_codes: Optional[torch.Tensor]
    q_scales: Optional[torch.Tensor]
    k_codes: Optional[torch.Tensor]
    k_scales: Optional[torch.Tensor]
    v_codes: Optional[torch.Tensor]
    v_scales: Optional[torch.Tensor]
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    d: int
    kv_stride: int
    scale_rule: int = SCALE_OCP  # block-scale rule the quantise / append calls write with


def alloc_mx(B, Hq, Hkv, Sq, kv_stride, d, device="cuda", scale_rule=0) -> MXQKV:
    """Output buffers of hifa4_quantize_qkv (uninitialised device memory)."""
    nblk = (kv_stride + 31) // 32
    u8 = dict(dtype=torch.uint8, device=device)
    return MXQKV(torch.empty((B, Hq, Sq, d // 2), **u8), torch.empty((B, Hq, Sq, d // 32), **u8),
                 torch.empty((B, Hkv, kv_stride, d // 2), **u8),
                 torch.empty((B, Hkv, kv_stride, d // 32), **u8),
                 torch.empty((B, Hkv, nblk, d, 16), **u8), torch.empty((B, Hkv, nblk, d), **u8),
                 B, Hq, Hkv, Sq, 0, d, kv_stride, int(scale_rule))


def _rope_struct(cos: torch.Tensor, sin: torch.Tensor, q_pos0: int, k_pos0: int) -> RopeC:
    if (cos.dtype != torch.float32 or sin.dtype != torch.float32 or cos.dim() != 2
            or cos.shape != sin.shape or not cos.is_contiguous() or not sin.is_contiguous()):
        raise ValueError("rope tables must be contiguous float32 [n_pos, d/2] of one shape")
    return RopeC(_ptr(cos), _ptr(sin), int(cos.shape[0]), int(q_pos0), int(k_pos0))


def hifa4_quantize_qkv(q: Optional[torch.Tensor], k: Optional[torch.Tensor],
                       v: Optional[torch.Tensor], smooth: Optional[torch.Tensor] = None, *,
                       kv_stride: int = 0, out: Optional[MXQKV] = None, Hkv: Optional[int] = None,
                       scale_rule: Optional[int] = None, stream=None) -> MXQKV:
    """Smooth-QK + MXFP4 quantisation; q [B,Hq,Sq,d], k/v [B,Hkv,Sk,d] bf16 or fp16 on the GPU.

    With k and v both None, pass Hkv (the smoothing rows are per KV head).  scale_rule
    (SCALE_OCP or SCALE_NOCLIP) is recorded in the returned tensors; None keeps out's rule
    (SCALE_OCP for new tensors).
    """
    return _quantize(q, k, v, smooth, None, kv_stride=kv_stride, out=out, Hkv=Hkv,
                     scale_rule=scale_rule, stream=stream)


def hifa4_quantize_qkv_rope(q: Optional[torch.Tensor], k: Optional[torch.Tensor],
                            v: Optional[torch.Tensor], cos: torch.Tensor, sin: torch.Tensor, *,
                            q_pos0: int = 0, k_pos0: int = 0,
                            smooth: Optional[torch.Tensor] = None, kv_stride: int = 0,
                            out: Optional[MXQKV] = None, Hkv: Optional[int] = None,
                            scale_rule: Optional[int] = None, stream=None) -> MXQKV:
    """hifa4_quantize_qkv after rotate-half RoPE of Q and K with the tables cos / sin
    (float32 [n_pos, d/2] on the GPU); query token t sits at position q_pos0 + t, key
    token t at k_pos0 + t."""
    rope = _rope_struct(cos, sin, q_pos0, k_pos0)
    return _quantize(q, k, v, smooth, rope, kv_stride=kv_stride, out=out, Hkv=Hkv,
                     scale_rule=scale_rule, stream=stream)


def _quantize(q, k, v, smooth, rope: Optional[RopeC], *, kv_stride, out, Hkv, scale_rule,
              stream) -> MXQKV:
    ref = next(t for t in (q, k, v) if t is not None)
    B, d = ref.shape[0], ref.shape[3]
    Hq, Sq = (q.shape[1], q.shape[2]) if q is not None else (1, 0)
    kk = k if k is not None else v
    if kk is not None:
        Hkv, Sk = kk.shape[1], kk.shape[2]
    else:
        Hkv, Sk = (Hkv if Hkv is not None else (smooth.shape[0] if smooth is not None else Hq)), 0
    if q is None:
        Hq = Hkv
    for t in (q, k, v):
        if t is not None and (t.dim() != 4 or t.dtype != ref.dtype):
            raise ValueError("q/k/v must be 4-d tensors of one dtype")
    cap = kv_stride or Sk
    if out is None:
        out = alloc_mx(B, Hq, Hkv, Sq, cap, d, device=ref.device)
    # only the shapes of the tensors given change (a K/V-only call keeps out's Q shape)
    if q is not None:
        out.Sq = Sq
    if kk is not None:
        out.Sk, out.kv_stride = Sk, cap
    if scale_rule is not None:
        out.scale_rule = int(scale_rule)
    r = out.scale_rule
    if smooth is not None and (smooth.dtype != torch.float32 or tuple(smooth.shape) != (Hkv, d)):
        raise ValueError("smooth must be float32 [Hkv, d]")
    if q is not None:
        _check_row_mx(out.q_codes, out.q_scales, B * Hq * Sq, d, "q")
    if k is not None:
        if tuple(k.shape) != (B, Hkv, Sk, d):
            raise ValueError("k must be [B, Hkv, Sk, d] = %s" % ((B, Hkv, Sk, d),))
        _check_row_mx(out.k_codes, out.k_scales, B * Hkv * cap, d, "k")
    if v is not None:
        if tuple(v.shape) != (B, Hkv, Sk, d):
            raise ValueError("v must be [B, Hkv, Sk, d] = %s" % ((B, Hkv, Sk, d),))
        _check_col_mx(out.v_codes, out.v_scales, B * Hkv, cap, d, "v")
    lib = load_library()
    mq = MxTensorC(_ptr(out.q_codes) if q is not None else None,
                   _ptr(out.q_scales) if q is not None else None, r)
    mk = MxTensorC(_ptr(out.k_codes) if k is not None else None,
                   _ptr(out.k_scales) if k is not None else None, r)
    mv = MxTensorC(_ptr(out.v_codes) if v is not None else None,
                   _ptr(out.v_scales) if v is not None else None, r)
    if rope is None:
        _check(lib.hifa4_quantize_qkv(_ptr(q), _ptr(k), _ptr(v), _dtype_code(ref.dtype), B, Hq,
                                      Hkv, Sq, Sk, kv_stride, d, _ptr(smooth), mq, mk, mv,
                                      _stream(stream)))
    else:
        _check(lib.hifa4_quantize_qkv_rope(_ptr(q), _ptr(k), _ptr(v), _dtype_code(ref.dtype), B,
                                           Hq, Hkv, Sq, Sk, kv_stride, d, _ptr(smooth),
                                           ctypes.byref(rope), mq, mk, mv, _stream(stream)))
    return out


def alloc_v_tail(B, Hkv, d, dtype=torch.bfloat16, device="cuda") -> torch.Tensor:
    """Zeroed raw-value tail buffer [B, Hkv, 32, d] of hifa4_kv_append."""
    return torch.zeros((B, Hkv, 32, d), dtype=dtype, device=device)


def hifa4_kv_append(q: Optional[torch.Tensor], k: torch.Tensor, v: torch.Tensor,
                    kv_lens: torch.Tensor, cache: MXQKV, v_tail: torch.Tensor, *,
                    kv_lens_out: Optional[torch.Tensor] = None,
                    smooth: Optional[torch.Tensor] = None, cos: Optional[torch.Tensor] = None,
                    sin: Optional[torch.Tensor] = None, q_pos0: int = 0, k_pos0: int = 0,
                    stream=None) -> MXQKV:
    """Append k / v [B,Hkv,n,d] to the MXFP4 cache at each sequence's length kv_lens
    (int32 [B] on the GPU) after RoPE (cos / sin, optional) and Smooth-QK; q [B,Hq,n,d]
    (optional) is quantised into cache.q_codes / q_scales at the same positions.
    kv_lens_out (int32 [B]) receives the new lengths.  Returns cache with Sq = n and
    Sk = its capacity (the upper bound the decode attention takes with kv_lens).  New blocks
    take cache.scale_rule."""
    if k.dim() != 4 or v.shape != k.shape or k.dtype != v.dtype:
        raise ValueError("k and v must be 4-d tensors of one shape and dtype")
    B, Hkv, n, d = k.shape
    Hq = q.shape[1] if q is not None else cache.Hq
    if q is not None and (tuple(q.shape) != (B, Hq, n, d) or q.dtype != k.dtype):
        raise ValueError("q must be [B, Hq, n, d] in k's dtype")
    if kv_lens.dtype != torch.int32 or kv_lens.numel() != B:
        raise ValueError("kv_lens must be int32 [B]")
    if kv_lens_out is not None and (kv_lens_out.dtype != torch.int32 or kv_lens_out.numel() != B):
        raise ValueError("kv_lens_out must be int32 [B]")
    if tuple(v_tail.shape) != (B, Hkv, 32, d) or v_tail.dtype != k.dtype:
        raise ValueError("v_tail must be [B, Hkv, 32, d] in k's dtype")
    if q is not None and tuple(cache.q_codes.shape) != (B, Hq, n, d // 2):
        raise ValueError("cache.q_codes must be [B, Hq, n, d/2]")
    if q is not None:
        _check_row_mx(cache.q_codes, cache.q_scales, B * Hq * n, d, "cache.q")
    if (cache.B, cache.Hkv, cache.d) != (B, Hkv, d):
        raise ValueError("cache is [B=%d, Hkv=%d, d=%d], k is [%d, %d, ., %d]"
                         % (cache.B, cache.Hkv, cache.d, B, Hkv, d))
    _check_row_mx(cache.k_codes, cache.k_scales, B * Hkv * cache.kv_stride, d, "cache.k")
    _check_col_mx(cache.v_codes, cache.v_scales, B * Hkv, cache.kv_stride, d, "cache.v")
    rope = None
    if cos is not None or sin is not None:
        if cos is None or sin is None:
            raise ValueError("give both rope tables or neither")
        rope = ctypes.byref(_rope_struct(cos, sin, q_pos0, k_pos0))
    r = cache.scale_rule
    mq = MxTensorC(_ptr(cache.q_codes), _ptr(cache.q_scales), r) if q is not None else MxTensorC()
    _check(load_library().hifa4_kv_append(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(k.dtype), B, Hq, Hkv, n, cache.kv_stride, d,
        _ptr(kv_lens), _ptr(kv_lens_out), _ptr(smooth), rope, _ptr(v_tail), mq,
        MxTensorC(_ptr(cache.k_codes), _ptr(cache.k_scales), r),
        MxTensorC(_ptr(cache.v_codes), _ptr(cache.v_scales), r), _stream(stream)))
    cache.Sq, cache.Sk = n, cache.kv_stride
    return cache


def hifa4_smooth_calibrate_workspace_size(Hkv: int, d: int) -> int:
    return int(load_library().hifa4_smooth_calibrate_workspace_size(int(Hkv), int(d)))


def hifa4_smooth_calibrate(q: torch.Tensor, k: torch.Tensor, alpha: float, *,
                           cos: Optional[torch.Tensor] = None, sin: Optional[torch.Tensor] = None,
                           q_pos0: int = 0, k_pos0: int = 0, out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """Smooth-QK factors s [Hkv, d] float32 from calibration activations q [B,Hq,S,d] and
    k [B,Hkv,S,d] (bf16 or fp16 on the GPU), rotated first by cos / sin when given."""
    if q.dim() != 4 or k.dim() != 4 or q.dtype != k.dtype:
        raise ValueError("q and k must be 4-d tensors of one dtype")
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, S, d):
        raise ValueError("k must be [B, Hkv, S, d] with q's B, S and d")
    if out is None:
        out = torch.empty((Hkv, d), dtype=torch.float32, device=q.device)
    if tuple(out.shape) != (Hkv, d) or out.dtype != torch.float32:
        raise ValueError("out must be float32 [Hkv, d]")
    need = hifa4_smooth_calibrate_workspace_size(Hkv, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    rope = None
    if cos is not None or sin is not None:
        if cos is None or sin is None:
            raise ValueError("give both rope tables or neither")
        rope = ctypes.byref(_rope_struct(cos, sin, q_pos0, k_pos0))
    _check(load_library().hifa4_smooth_calibrate(
        _ptr(q), _ptr(k), _dtype_code(q.dtype), B, Hq, Hkv, S, d, rope, float(alpha), _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def make_params(B, Hq, Hkv, Sq, Sk, d, *, causal, sm_scale=None, kv_stride=0, kv_lens=None,
                decode_chunk=0, rescale_threshold=0.0, normaliser=0,
                scale_rule=0) -> AttnParamsC:
    return AttnParamsC(B, Hq, Hkv, Sq, Sk, d, 1 if causal else 0,
                       float(sm_scale) if sm_scale else 0.0, kv_stride,
                       _ptr(kv_lens) if kv_lens is not None else None, decode_chunk,
                       float(rescale_threshold), int(normaliser), int(scale_rule))


def hifa4_attn_workspace_size(params: AttnParamsC) -> int:
    return int(load_library().hifa4_attn_workspace_size(ctypes.byref(params)))


def hifa4_attn_schedule(params: AttnParamsC) -> tuple[int, int]:
    bn, ch = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load_library().hifa4_attn_schedule(ctypes.byref(params), ctypes.byref(bn),
                                              ctypes.byref(ch)))
    return bn.value, ch.value


def hifa4_attn_decode_piece_tiles(params: AttnParamsC, total_tiles: int) -> int:
    return int(load_library().hifa4_attn_decode_piece_tiles(ctypes.byref(params), int(total_tiles)))


def hifa4_attn_fwd(mx: MXQKV, *, causal: bool, sm_scale: Optional[float] = None,
                   kv_lens: Optional[torch.Tensor] = None, decode_chunk: int = 0,
                   out: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16,
                   lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                   workspace: Optional[torch.Tensor] = None, rescale_threshold: float = 0.0,
                   normaliser: int = 0, scale_rule: int = SCALE_OCP, stream=None):
    """Fused MXFP4 attention on quantised operands; returns (out, lse or None).
    scale_rule: block-scale rule of P_hat."""
    if kv_lens is not None and (kv_lens.dtype != torch.int32 or kv_lens.numel() != mx.B):
        raise ValueError("kv_lens must be int32 [B]")
    p = make_params(mx.B, mx.Hq, mx.Hkv, mx.Sq, mx.Sk, mx.d, causal=causal, sm_scale=sm_scale,
                    kv_stride=mx.kv_stride, kv_lens=kv_lens, decode_chunk=decode_chunk,
                    rescale_threshold=rescale_threshold, normaliser=normaliser,
                    scale_rule=scale_rule)
    dev = mx.q_codes.device
    if out is None:
        out = torch.empty((mx.B, mx.Hq, mx.Sq, mx.d), dtype=out_dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((mx.B, mx.Hq, mx.Sq), dtype=torch.float32, device=dev)
    _check_out_lse(out, lse, mx.B, mx.Hq, mx.Sq, mx.d)
    _check_row_mx(mx.q_codes, mx.q_scales, mx.B * mx.Hq * mx.Sq, mx.d, "q")
    cap = mx.kv_stride or mx.Sk
    if cap:
        _check_row_mx(mx.k_codes, mx.k_scales, mx.B * mx.Hkv * cap, mx.d, "k")
        _check_col_mx(mx.v_codes, mx.v_scales, mx.B * mx.Hkv, cap, mx.d, "v")
    need = hifa4_attn_workspace_size(p)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if need:
        _need_bytes(workspace, need, "workspace")
    lib = load_library()
    _check(lib.hifa4_attn_fwd(ctypes.byref(p), MxTensorC(_ptr(mx.q_codes), _ptr(mx.q_scales)),
                              MxTensorC(_ptr(mx.k_codes), _ptr(mx.k_scales)),
                              MxTensorC(_ptr(mx.v_codes), _ptr(mx.v_scales)), _ptr(out),
                              _dtype_code(out.dtype), _ptr(lse), _ptr(workspace),
                              workspace.numel() if workspace is not None else 0,
                              _stream(stream)))
    return out, lse


def hifa4_attn_fwd_noalloc(mx: MXQKV, *, causal: bool, sm_scale: Optional[float] = None,
                           kv_lens: Optional[torch.Tensor] = None, decode_chunk: int = 0,
                           out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                           rescale_threshold: float = 0.0, normaliser: int = 0,
                           scale_rule: int = SCALE_OCP, stream=None):
    """hifa4_attn_fwd with the decode partials in the library's own device scratch: the
    caller passes every buffer (out, and lse or None) and nothing is allocated.  Calls that
    overlap on one GPU share that scratch and must be serialised by the caller."""
    if kv_lens is not None and (kv_lens.dtype != torch.int32 or kv_lens.numel() != mx.B):
        raise ValueError("kv_lens must be int32 [B]")
    p = make_params(mx.B, mx.Hq, mx.Hkv, mx.Sq, mx.Sk, mx.d, causal=causal, sm_scale=sm_scale,
                    kv_stride=mx.kv_stride, kv_lens=kv_lens, decode_chunk=decode_chunk,
                    rescale_threshold=rescale_threshold, normaliser=normaliser,
                    scale_rule=scale_rule)
    _check_out_lse(out, lse, mx.B, mx.Hq, mx.Sq, mx.d)
    _check_row_mx(mx.q_codes, mx.q_scales, mx.B * mx.Hq * mx.Sq, mx.d, "q")
    cap = mx.kv_stride or mx.Sk
    if cap:
        _check_row_mx(mx.k_codes, mx.k_scales, mx.B * mx.Hkv * cap, mx.d, "k")
        _check_col_mx(mx.v_codes, mx.v_scales, mx.B * mx.Hkv, cap, mx.d, "v")
    _check(load_library().hifa4_attn_fwd_noalloc(
        ctypes.byref(p), MxTensorC(_ptr(mx.q_codes), _ptr(mx.q_scales)),
        MxTensorC(_ptr(mx.k_codes), _ptr(mx.k_scales)),
        MxTensorC(_ptr(mx.v_codes), _ptr(mx.v_scales)), _ptr(out), _dtype_code(out.dtype),
        _ptr(lse), _stream(stream)))
    return out, lse


def hifa4_attn_fwd_qraw(q: torch.Tensor, smooth: Optional[torch.Tensor], mx: MXQKV, *,
                        causal: bool, sm_scale: Optional[float] = None,
                        out: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16,
                        lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                        rescale_threshold: float = 0.0, normaliser: int = 0,
                        scale_rule: int = SCALE_OCP, stream=None):
    """Prefill with Q as bf16 / fp16 activations [B,Hq,Sq,d], smoothed and quantised inside
    the kernel; mx holds the quantised K and V (its Q fields are not read).  scale_rule
    governs both P_hat and the in-kernel Q blocks.
    Returns (out, lse or None)."""
    B, Hq, Sq, d = q.shape
    if q.dtype not in (torch.bfloat16, torch.float16) or not q.is_contiguous():
        raise ValueError("q must be a contiguous bf16 / fp16 tensor")
    if (B, Hq, d) != (mx.B, mx.Hq, mx.d):
        raise ValueError("q does not match the MX tensors")
    if smooth is not None and (smooth.dtype != torch.float32 or tuple(smooth.shape) != (mx.Hkv, d)):
        raise ValueError("smooth must be float32 [Hkv, d]")
    p = make_params(B, Hq, mx.Hkv, Sq, mx.Sk, d, causal=causal, sm_scale=sm_scale,
                    kv_stride=mx.kv_stride, rescale_threshold=rescale_threshold,
                    normaliser=normaliser, scale_rule=scale_rule)
    if out is None:
        out = torch.empty((B, Hq, Sq, d), dtype=out_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    _check_out_lse(out, lse, B, Hq, Sq, d)
    cap = mx.kv_stride or mx.Sk
    if cap:
        _check_row_mx(mx.k_codes, mx.k_scales, B * mx.Hkv * cap, d, "k")
        _check_col_mx(mx.v_codes, mx.v_scales, B * mx.Hkv, cap, d, "v")
    _check(load_library().hifa4_attn_fwd_qraw(
        ctypes.byref(p), _ptr(q), _dtype_code(q.dtype), _ptr(smooth),
        MxTensorC(_ptr(mx.k_codes), _ptr(mx.k_scales)), MxTensorC(_ptr(mx.v_codes), _ptr(mx.v_scales)),
        _ptr(out), _dtype_code(out.dtype), _ptr(lse), None, 0, _stream(stream)))
    return out, lse


def bf16_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool,
                  sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                  rescale_threshold: float = 0.0, stream=None):
    """bf16 FlashAttention baseline; q [B,Hq,Sq,d], k/v [B,Hkv,Sk,d] bf16; returns (out, lse)."""
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    for t in (q, k, v):
        if t.dtype != torch.bfloat16:
            raise ValueError("bf16_attn_fwd takes bfloat16 tensors")
    if tuple(k.shape) != (B, Hkv, Sk, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must both be [B, Hkv, Sk, d] with q's B and d")
    p = make_params(B, Hq, Hkv, Sq, Sk, d, causal=causal, sm_scale=sm_scale,
                    rescale_threshold=rescale_threshold)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    _need_shape(out, (B, Hq, Sq, d), (torch.bfloat16,), "out")
    if lse is not None:
        _need_shape(lse, (B, Hq, Sq), (torch.float32,), "lse")
    _check(load_library().bf16_attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                        _ptr(lse), None, 0, _stream(stream)))
    return out, lse
