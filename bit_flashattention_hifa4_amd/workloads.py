"""Seeded synthetic workloads for the attention path.

This module only makes inputs: it holds none of the attention path's
arithmetic (no quantisation, no softmax, no attention).  Both the HIP path and
the CPU oracle receive exactly the tensors made here.  Its RoPE and its
calibration of s are part of the input recipe (they make synthetic post-RoPE
activations and a static smoothing vector); the library's own RoPE and
calibration are checked against the oracle's, never against these.

The pages measure HiFA4 on activation traces of real LLMs (Qwen3-8B, Gemma2-9B,
Llama-3.1-8B, Mistral-7B, Phi-4B; "HiFA4: Training-Free 4-bit FlashAttention on
Ascend HIF4 NPUs for LLM Inference", Abstract).  Those weights and traces are
not available, so the workloads below stand in for them with the same head
counts, head dims and sequence lengths, N(0, 1) activations, a synthetic RoPE,
and seeded outlier key channels (the situation Smooth-QK is meant for: it
moves quantisation difficulty from K to Q, Abstract, Smooth-QK).

Recipe (per config):
  * numpy ``default_rng`` (PCG64), float32 standard normals;
  * RoPE (rotate-half pairs (j, j + d/2), inverse frequency theta^(-2j/d),
    positions 0..S-1) applied in float32 to Q and K when the config names a
    theta;
  * outlier key channels (seeded, per KV head) multiplied by a factor, after
    RoPE, because Smooth-QK acts on post-RoPE keys;
  * cast to bf16 / fp16 with round-to-nearest-even (torch CPU);
  * the smoothing vector s (calibration-static, per KV head and channel) is
    computed offline from a separate seeded 512-token calibration sample
    drawn with the same recipe, as the config states:
    s_j = (max|K_j| / max|Q_j|)^alpha, the maxima taken over the calibration
    tokens (and over all query heads of the KV head's group), in float64, then
    rounded to float32; a zero maximum gives s_j = 1.  s is an *input* of the
    attention path, exactly like Q, K and V.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

BASE_SEED = 20260705


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    S: int
    d: int
    causal: bool
    dtype: str                      # "bf16" or "fp16"
    rope_theta: Optional[float]
    n_outliers: int                 # outlier K channels per KV head
    outlier_factor: float
    fixed_outliers: tuple = ()      # explicit outlier channels (tiny config)
    smooth_alpha: Optional[float] = None   # None: s = 1 (Smooth-QK off)
    calib_tokens: int = 0           # 0: calibrate on the inputs themselves
    seed: int = BASE_SEED

    @property
    def Sq(self) -> int:
        return self.S

    @property
    def Sk(self) -> int:
        return self.S

    def flops(self) -> float:
        """Algorithmic flops: 4 d per unmasked (query, key) pair, per batch and query head."""
        if self.causal:
            pairs = self.S * (self.S + 1) // 2
        else:
            pairs = self.S * self.S
        return 4.0 * self.d * pairs * self.B * self.Hq


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    min_len: int
    max_len: int
    dtype: str = "bf16"
    seed: int = BASE_SEED + 500


# The five workloads.  The first is the small case the oracle finishes in
# seconds; the Gemma2-9B-shaped causal prefill, the largest, is the benchmark's
# headline, and the other prefill shapes and the decode cache are its legs.
TINY = PrefillConfig("tiny_b1_h1_s128_d64", 1, 1, 1, 128, 64, False, "fp16", None, 0, 8.0,
                     fixed_outliers=(3, 17), smooth_alpha=0.5, calib_tokens=0,
                     seed=BASE_SEED + 100)
QWEN3_8B = PrefillConfig("qwen3_8b_prefill_b1_hq32_hkv8_s4096_d128", 1, 32, 8, 4096, 128, True,
                         "bf16", 1.0e6, 4, 10.0, smooth_alpha=0.5, calib_tokens=512,
                         seed=BASE_SEED + 200)
LLAMA31_8B = PrefillConfig("llama31_8b_prefill_b8_hq32_hkv8_s2048_d128", 8, 32, 8, 2048, 128,
                           True, "bf16", 5.0e5, 0, 1.0, smooth_alpha=None,
                           seed=BASE_SEED + 300)
GEMMA2_9B = PrefillConfig("gemma2_9b_prefill_b4_hq16_hkv8_s4096_d256", 4, 16, 8, 4096, 256, True,
                          "bf16", None, 2, 6.0, smooth_alpha=0.25, calib_tokens=512,
                          seed=BASE_SEED + 400)
DECODE = DecodeConfig("decode_b64_hq32_hkv8_d128_len1k_32k", 64, 32, 8, 128, 1024, 32768)

PREFILL_CONFIGS = {c.name: c for c in (TINY, QWEN3_8B, LLAMA31_8B, GEMMA2_9B)}


def _torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "fp16": torch.float16}[name]


def rope_tables(n_pos: int, d: int, theta: float):
    """cos / sin tables float32 [n_pos, d/2] of the standard rotary frequencies
    theta^(-2j/d), angles computed in fp64 and rounded once."""
    half = d // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def apply_rope(x: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE on [..., S, d] float32, positions 0..S-1."""
    S, d = x.shape[-2], x.shape[-1]
    half = d // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = np.arange(S, dtype=np.float64)[:, None] * inv[None, :]
    cos = np.cos(ang).astype(np.float32)
    sin = np.sin(ang).astype(np.float32)
    a = x[..., :half]
    b = x[..., half:]
    out = np.empty_like(x)
    out[..., :half] = a * cos - b * sin
    out[..., half:] = b * cos + a * sin
    return out


def outlier_channels(cfg: PrefillConfig) -> np.ndarray:
    """[Hkv, n] channel indices of the outlier key channels (same for calibration data)."""
    if cfg.fixed_outliers:
        return np.tile(np.asarray(cfg.fixed_outliers, dtype=np.int64), (cfg.Hkv, 1))
    if cfg.n_outliers == 0:
        return np.zeros((cfg.Hkv, 0), dtype=np.int64)
    rng = np.random.default_rng(cfg.seed + 2)
    return np.stack([rng.choice(cfg.d, size=cfg.n_outliers, replace=False)
                     for _ in range(cfg.Hkv)])


def _draw_qkv(cfg: PrefillConfig, seed: int, B: int, S: int):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, cfg.Hq, S, cfg.d), dtype=np.float32)
    k = rng.standard_normal((B, cfg.Hkv, S, cfg.d), dtype=np.float32)
    v = rng.standard_normal((B, cfg.Hkv, S, cfg.d), dtype=np.float32)
    if cfg.rope_theta is not None:
        q = apply_rope(q, cfg.rope_theta)
        k = apply_rope(k, cfg.rope_theta)
    ch = outlier_channels(cfg)
    for g in range(cfg.Hkv):
        if ch.shape[1]:
            k[:, g, :, ch[g]] *= np.float32(cfg.outlier_factor)
    dt = _torch_dtype(cfg.dtype)
    return (torch.from_numpy(q).to(dt), torch.from_numpy(k).to(dt), torch.from_numpy(v).to(dt))


def calibrate_smooth(q: torch.Tensor, k: torch.Tensor, alpha: float) -> np.ndarray:
    """Offline calibration of s [Hkv, d] from calibration activations (see module doc)."""
    qf = q.double().abs()
    kf = k.double().abs()
    B, Hq, S, d = qf.shape
    Hkv = kf.shape[1]
    g = Hq // Hkv
    qmax = qf.reshape(B, Hkv, g, S, d).amax(dim=(0, 2, 3)).numpy()
    kmax = kf.amax(dim=(0, 2)).numpy()
    with np.errstate(divide="ignore", invalid="ignore"):
        s = np.where((qmax > 0) & (kmax > 0), (kmax / np.where(qmax > 0, qmax, 1.0)) ** alpha, 1.0)
    return s.astype(np.float32)


def prefill_inputs(cfg: PrefillConfig):
    """Returns dict(q, k, v: torch CPU tensors [B,H,S,d] in cfg.dtype; smooth: float32 [Hkv,d] or None)."""
    q, k, v = _draw_qkv(cfg, cfg.seed, cfg.B, cfg.S)
    smooth = None
    if cfg.smooth_alpha is not None:
        if cfg.calib_tokens:
            cq, ck, _ = _draw_qkv(cfg, cfg.seed + 1, 1, cfg.calib_tokens)
        else:
            cq, ck = q, k
        smooth = calibrate_smooth(cq, ck, cfg.smooth_alpha)
    return dict(q=q, k=k, v=v, smooth=smooth)


def random_case(B, Hq, Hkv, Sq, Sk, d, *, dtype="bf16", seed=0, rope_theta=None,
                n_outliers=0, outlier_factor=8.0, smooth_alpha=None, scale=1.0):
    """Small seeded case with arbitrary shapes (ragged lengths, Sq != Sk) for parity tests."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Sq, d), dtype=np.float32) * np.float32(scale)
    k = rng.standard_normal((B, Hkv, Sk, d), dtype=np.float32) * np.float32(scale)
    v = rng.standard_normal((B, Hkv, Sk, d), dtype=np.float32)
    if rope_theta is not None:
        q = apply_rope(q, rope_theta)
        k = apply_rope(k, rope_theta)
    if n_outliers:
        for g in range(Hkv):
            ch = rng.choice(d, size=n_outliers, replace=False)
            k[:, g, :, ch] *= np.float32(outlier_factor)
    dt = _torch_dtype(dtype)
    qt, kt, vt = (torch.from_numpy(a).to(dt) for a in (q, k, v))
    smooth = calibrate_smooth(qt, kt, smooth_alpha) if smooth_alpha is not None else None
    return dict(q=qt, k=kt, v=vt, smooth=smooth)


# --------------------------------------------------------------------------
# Decode against a long cache
# --------------------------------------------------------------------------

def decode_lengths(cfg: DecodeConfig = DECODE) -> np.ndarray:
    rng = np.random.default_rng(BASE_SEED)
    return rng.integers(cfg.min_len, cfg.max_len, size=cfg.B, endpoint=True).astype(np.int32)


def decode_q(cfg: DecodeConfig = DECODE) -> torch.Tensor:
    rng = np.random.default_rng(cfg.seed)
    q = rng.standard_normal((cfg.B, cfg.Hq, 1, cfg.d), dtype=np.float32)
    return torch.from_numpy(q).to(_torch_dtype(cfg.dtype))


def decode_kv(cfg: DecodeConfig, b: int, length: int):
    """K, V of sequence b: torch [1, Hkv, length, d]; reproducible per sequence."""
    rng = np.random.default_rng(cfg.seed + 1000 + b)
    k = rng.standard_normal((1, cfg.Hkv, length, cfg.d), dtype=np.float32)
    v = rng.standard_normal((1, cfg.Hkv, length, cfg.d), dtype=np.float32)
    dt = _torch_dtype(cfg.dtype)
    return torch.from_numpy(k).to(dt), torch.from_numpy(v).to(dt)


def to_f32(t: torch.Tensor) -> np.ndarray:
    """Exact float32 values of a bf16 / fp16 tensor."""
    return t.float().numpy()
