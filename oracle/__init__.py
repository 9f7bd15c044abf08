"""CPU oracle for HiFA4-style MXFP4 FlashAttention (test infrastructure).

Only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The product path never does: it runs
the HIP library and fails loudly if that library is missing.

The arithmetic lives in ``hifa4_oracle.c`` (plain C, fp64, pthreads), built
with gcc into ``libhifa4_oracle.so`` beside it.  This module only marshals
numpy arrays.  What each function follows is documented in the C file:
the HiFA4 abstract ("HiFA4: Training-Free 4-bit FlashAttention on Ascend HIF4
NPUs for LLM Inference") for Smooth-QK, P-Reordering, the online-softmax state
and the inconsistent-normaliser statistic, and the OCP MX v1.0 MXFP4 format as
the stated stand-in for the undefined HIF4 layout.

Every function here is pinned by ``tests/test_oracle_*.py`` against values the
pages or the mathematics fix (hand-worked codes, brute-force softmax attention,
closed forms and invariants); see those tests for which pin covers which part.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hifa4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libhifa4_oracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_F = ctypes.POINTER(ctypes.c_float)
_U8 = ctypes.POINTER(ctypes.c_uint8)
_I32 = ctypes.POINTER(ctypes.c_int32)
_I64 = ctypes.POINTER(ctypes.c_int64)


class _AttnCfg(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int),
        ("Sq", ctypes.c_int), ("Sk", ctypes.c_int), ("d", ctypes.c_int),
        ("causal", ctypes.c_int), ("sm_scale", ctypes.c_double),
        ("bc", ctypes.c_int), ("chunk", ctypes.c_int), ("quant_p", ctypes.c_int),
        ("br", ctypes.c_int), ("nthreads", ctypes.c_int), ("tau", ctypes.c_double),
        ("p_rule", ctypes.c_int), ("p_shift", ctypes.c_double),
    ]


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-pthread",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    _lib = _open(_LIB_PATH)
    return _lib


@contextlib.contextmanager
def use_library(path: str):
    """Temporarily route every call to another build of the oracle (mutation tests)."""
    global _lib
    saved = _lib
    _lib = _open(path)
    try:
        yield
    finally:
        _lib = saved


def _open(path: str):
    lib = ctypes.CDLL(path)
    lib.oracle_e2m1_value.restype = ctypes.c_double
    lib.oracle_e2m1_value.argtypes = [ctypes.c_uint]
    lib.oracle_e2m1_encode.restype = ctypes.c_uint
    lib.oracle_e2m1_encode.argtypes = [ctypes.c_double]
    lib.oracle_e2m1_encode_array.restype = None
    lib.oracle_e2m1_encode_array.argtypes = [_D, ctypes.c_long, _U8]
    lib.oracle_mx_block.restype = ctypes.c_uint
    lib.oracle_mx_block.argtypes = [_D, ctypes.c_int, ctypes.c_long, _U8, _D, ctypes.c_long,
                                    ctypes.c_int]
    lib.oracle_quantize_rows.restype = None
    lib.oracle_quantize_rows.argtypes = [_F, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, _F, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, _U8, _U8, _D, ctypes.c_int]
    lib.oracle_quantize_v.restype = None
    lib.oracle_quantize_v.argtypes = [_F, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, _U8, _U8, _D,
                                      ctypes.c_int]
    lib.oracle_rope_rows.restype = None
    lib.oracle_rope_rows.argtypes = [_F, ctypes.c_long, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     _F, _F, _F]
    lib.oracle_smooth_calibrate.restype = None
    lib.oracle_smooth_calibrate.argtypes = [_D, _D, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_double, _F]
    lib.oracle_eps_tiles.restype = None
    lib.oracle_eps_tiles.argtypes = [_D, _D, _D, _D, ctypes.c_long, _D, _D]
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_attention.argtypes = [ctypes.POINTER(_AttnCfg), _D, _D, _D, _I32, _I32, _I64,
                                     ctypes.c_long, _D, _D, _D, _D, _D, _D, _D, _D, _D, _D]
    return lib


def _ptr(a, typ):
    if a is None:
        return ctypes.cast(None, typ)
    return a.ctypes.data_as(typ)


def _f32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def default_threads() -> int:
    """Host threads for the oracle: OMP_NUM_THREADS when set (the CPU share), else all cores."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return max(1, os.cpu_count() or 1)


# --------------------------------------------------------------------------
# E2M1 / MX block
# --------------------------------------------------------------------------

def e2m1_value(code: int) -> float:
    return float(_load().oracle_e2m1_value(int(code)))


def e2m1_encode(y: float) -> int:
    return int(_load().oracle_e2m1_encode(float(y)))


def e2m1_encode_array(y) -> np.ndarray:
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float64))
    out = np.zeros(y.size, dtype=np.uint8)
    _load().oracle_e2m1_encode_array(_ptr(y, _D), y.size, _ptr(out, _U8))
    return out.reshape(y.shape)


def mx_block(x, rule: int = 0) -> tuple[np.ndarray, int, np.ndarray]:
    """Quantise one block of <= 32 values: (codes 0..15 per element, E8M0 byte, dequantised).

    rule 0: OCP MX shared exponent; rule 1: no-clip (one higher when amax > 6 * 2^e)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    n = x.size
    codes = np.zeros(n, dtype=np.uint8)
    deq = np.zeros(n, dtype=np.float64)
    sc = _load().oracle_mx_block(_ptr(x, _D), n, 1, _ptr(codes, _U8), _ptr(deq, _D), 1,
                                 int(rule))
    return codes, int(sc), deq


# --------------------------------------------------------------------------
# Smooth-QK + MXFP4 quantisation in the library's byte layouts
# --------------------------------------------------------------------------

def quantize_rows(x, smooth=None, *, divide: bool, cap: int | None = None,
                  quantise: bool = True, rule: int = 0):
    """Q (divide=False) or K (divide=True) rows: x fp32 [B,H,S,d]; smooth [Hs,d] or None.

    Returns (codes [B,H,cap,d/2] u8, scales [B,H,cap,d/32] u8, deq [B,H,S,d] f64).
    With quantise=False, deq holds the smoothed fp32 values and codes/scales are None.
    """
    x = _f32(x)
    B, H, S, d = x.shape
    cap = S if cap is None else cap
    group = 1
    sm = None
    if smooth is not None:
        sm = _f32(smooth)
        group = H // sm.shape[0]
        assert sm.shape == (H // group, d) and H % sm.shape[0] == 0
    deq = np.zeros((B, H, S, d), dtype=np.float64)
    codes = scales = None
    if quantise:
        assert d % 32 == 0
        codes = np.zeros((B, H, cap, d // 2), dtype=np.uint8)
        scales = np.zeros((B, H, cap, d // 32), dtype=np.uint8)
    _load().oracle_quantize_rows(_ptr(x, _F), B, H, S, d, _ptr(sm, _F), group, int(divide),
                                 cap, int(quantise), _ptr(codes, _U8), _ptr(scales, _U8),
                                 _ptr(deq, _D), int(rule))
    return codes, scales, deq


def quantize_v(x, *, cap: int | None = None, quantise: bool = True, rule: int = 0):
    """V: x fp32 [B,H,S,d] -> (codes [B,H,nblk,d,16], scales [B,H,nblk,d], deq [B,H,S,d])."""
    x = _f32(x)
    B, H, S, d = x.shape
    cap = S if cap is None else cap
    nblk = (cap + 31) // 32
    deq = np.zeros((B, H, S, d), dtype=np.float64)
    codes = scales = None
    if quantise:
        codes = np.zeros((B, H, nblk, d, 16), dtype=np.uint8)
        scales = np.zeros((B, H, nblk, d), dtype=np.uint8)
    _load().oracle_quantize_v(_ptr(x, _F), B, H, S, d, cap, int(quantise), _ptr(codes, _U8),
                              _ptr(scales, _U8), _ptr(deq, _D), int(rule))
    return codes, scales, deq


# --------------------------------------------------------------------------
# RoPE and the offline Smooth-QK calibration (the steps before the path)
# --------------------------------------------------------------------------

def rope_rows(x, cos, sin, pos0: int = 0):
    """Rotate-half RoPE of x [..., S, d] (fp32) with caller tables cos / sin [n_pos, d/2]
    (fp32); token t of every row group sits at position pos0 + t.  Returns fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    cos = np.ascontiguousarray(cos, dtype=np.float32)
    sin = np.ascontiguousarray(sin, dtype=np.float32)
    S, d = x.shape[-2], x.shape[-1]
    assert d % 2 == 0 and cos.shape == sin.shape and cos.shape[1] == d // 2
    assert 0 <= pos0 and pos0 + S <= cos.shape[0]
    out = np.empty_like(x)
    rows = x.size // d
    _load().oracle_rope_rows(_ptr(x, _F), rows, S, d, int(pos0), _ptr(cos, _F), _ptr(sin, _F),
                             _ptr(out, _F))
    return out


def smooth_calibrate(q, k, alpha: float):
    """s [Hkv, d] float32 from calibration activations q [B,Hq,S,d], k [B,Hkv,S,d]."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, S, d) and Hq % Hkv == 0
    s = np.empty((Hkv, d), dtype=np.float32)
    _load().oracle_smooth_calibrate(_ptr(q, _D), _ptr(k, _D), B, Hq, Hkv, S, d, float(alpha),
                                    _ptr(s, _F))
    return s


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def attention(q, k, v, *, causal: bool, sm_scale: float | None = None, bc: int = 64,
              chunk: int = 0, quant_p: bool = True, br: int = 128, kv_lens=None, rows=None,
              chunk_phase=None,
              want_weights: bool = False, want_eps: bool = False, nthreads: int | None = None,
              tau: float = 0.0, p_rule: int = 0, p_shift: float = 0.0):
    """Online-softmax attention over dequantised (or exact) operands, fp64.

    q [B,Hq,Sq,d]; k, v [B,Hkv,Sk,d] (float64).  tau: lazy-rescale threshold
    (log2 units, 0 = FlashAttention-2 frame).  p_rule: block-scale rule of
    P_hat (0 OCP, 1 no-clip).  p_shift (log2 units, normally 0): P is taken as
    exp(S - m) * 2^p_shift, which leaves exact attention unchanged and moves
    P_hat's decisions only for P within 2^|p_shift| of a boundary of the 4-bit
    format (see the C source).  chunk > 0 splits each row's keys
    into runs that start from a fresh softmax state and are merged with the
    log-sum-exp rule; chunk_phase [B,Hkv] (keys, multiples of bc below chunk)
    shifts that grid: a run starts at every key t > 0 with (t + phase) % chunk
    == 0.  Returns a dict with
    o, o_naive, l, l_naive, lse (and w, eps_* when asked).  With ``rows`` (flat
    ids (b*Hq + h)*Sq + i) only those rows are computed, in that order.
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    B, Hq, Sq, d = q.shape
    _, Hkv, Sk, _ = k.shape
    cfg = _AttnCfg(B, Hq, Hkv, Sq, Sk, d, int(causal),
                   float(sm_scale if sm_scale is not None else 1.0 / np.sqrt(d)),
                   int(bc), int(chunk), int(quant_p), int(br),
                   int(nthreads or default_threads()), float(tau), int(p_rule), float(p_shift))
    lens = None
    if kv_lens is not None:
        lens = np.ascontiguousarray(np.asarray(kv_lens, dtype=np.int32))
        assert lens.shape == (B,) and (lens <= Sk).all()
    ph = None
    if chunk_phase is not None:
        ph = np.ascontiguousarray(np.asarray(chunk_phase, dtype=np.int32))
        assert ph.shape == (B, Hkv)
    rr = None
    n = B * Hq * Sq
    if rows is not None:
        rr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rr.size
    o = np.zeros((n, d))
    o_naive = np.zeros((n, d))
    lse = np.zeros(n)
    l = np.zeros(n)
    ln = np.zeros(n)
    w = np.zeros((n, Sk)) if want_weights else None
    eps = None
    if want_eps and rows is None:
        n_qt = -(-Sq // br)
        n_kt = -(-Sk // bc)
        eps = [np.zeros((B, Hq, n_qt, n_kt)) for _ in range(4)]
    e = eps or [None] * 4
    rc = _load().oracle_attention(ctypes.byref(cfg), _ptr(q, _D), _ptr(k, _D), _ptr(v, _D),
                                  _ptr(lens, _I32), _ptr(ph, _I32), _ptr(rr, _I64), n, _ptr(o, _D),
                                  _ptr(lse, _D), _ptr(o_naive, _D), _ptr(l, _D), _ptr(ln, _D),
                                  _ptr(w, _D), _ptr(e[0], _D), _ptr(e[1], _D), _ptr(e[2], _D),
                                  _ptr(e[3], _D))
    if rc != 0:
        raise ValueError("oracle_attention: bad configuration")
    shape = (B, Hq, Sq) if rows is None else (n,)
    out = dict(o=o.reshape(shape + (d,)), o_naive=o_naive.reshape(shape + (d,)),
               lse=lse.reshape(shape), l=l.reshape(shape), l_naive=ln.reshape(shape))
    if w is not None:
        out["w"] = w.reshape(shape + (Sk,))
    if eps is not None:
        mean = np.zeros_like(eps[0])
        pooled = np.zeros_like(eps[0])
        _load().oracle_eps_tiles(_ptr(eps[0], _D), _ptr(eps[1], _D), _ptr(eps[2], _D),
                                 _ptr(eps[3], _D), eps[0].size, _ptr(mean, _D),
                                 _ptr(pooled, _D))
        out["eps_tile_mean"] = mean
        out["eps_tile_pooled"] = pooled
        out["eps_tile_rows"] = eps[1]
    return out


def quantize_qkv(q, k, v, smooth=None, *, kv_cap: int | None = None, rule: int = 0):
    """Smooth-QK + MXFP4 of all three operands, in the library's layouts.

    q [B,Hq,Sq,d], k/v [B,Hkv,Sk,d] fp32 (exact values of the bf16/fp16 inputs).
    Returns dict: q_codes, q_scales, q_deq, k_codes, k_scales, k_deq, v_codes,
    v_scales, v_deq.
    """
    out = {}
    if q is not None:
        out["q_codes"], out["q_scales"], out["q_deq"] = quantize_rows(q, smooth, divide=False,
                                                                      rule=rule)
    if k is not None:
        out["k_codes"], out["k_scales"], out["k_deq"] = quantize_rows(k, smooth, divide=True,
                                                                      cap=kv_cap, rule=rule)
    if v is not None:
        out["v_codes"], out["v_scales"], out["v_deq"] = quantize_v(v, cap=kv_cap, rule=rule)
    return out
