#!/usr/bin/env python3
"""Benchmark of the MXFP4 FlashAttention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline workload: the Gemma2-9B-shaped causal prefill layer (B=4, 16 query
heads, 8 KV heads, d=256, S=4096, bf16 inputs, 2 outlier key channels per
head, mild calibration-static smoothing), the largest prefill configuration
that runs on one GPU.  One step is one pass of the whole hot path over that
batch, inputs resident in HBM: Smooth-QK + MXFP4 quantisation of K and V (one
launch), then the fused MXFP4 attention, which smooths and quantises its own Q
rows in its prologue (one launch; the codes are bit-identical to quantising Q
separately).  `value` = algorithmic attention flops (4 d per unmasked
query-key pair) per second of step time.

The attention runs with the lazy-rescale threshold 8 (log2 units; the running
max moves only when a tile's max exceeds it by more than that, and P_hat is
defined in that frame; the CPU oracle takes the same value).

Also reported (in "extra"): the same step on the Qwen3-8B- and Llama-3.1-8B-
shaped prefill layers (the other prefill configurations, each timed here and
put against the FP4 peak and against the measured pure-MFMA rate), the step's
kernels one by one, the unfused step (Q, K, V quantised in one launch,
attention on Q codes), the attention with threshold 0 (the FlashAttention-2
frame), with the pages' non-reordered normaliser and under the no-clip
block-scale rule, the bf16 FlashAttention baseline (time ratio = the measured
counterpart of the pages' projected latency cut), the attention kernel at
8k-32k tokens, the split-K decode on 64 sequences with 1k-32k MXFP4 cache
entries (HBM GB/s, split + merge, rotating over three copies of the cache),
the decode step (one-token cache append + attention), the HBM read rate of a
plain streaming kernel and the FP4 MFMA rate of a pure-MFMA kernel.  The
accuracy of the headline output on a sample (every row of batch entry 0)
against fp64 exact attention and against the oracle, and the oracle's
per-tile normaliser-mismatch statistic on that sample, come with the CPU
baseline.

Every timed region follows at least 200 ms of untimed launches of the same
work (the GPU's clocks ramp up under sustained load), then the W warm-up
steps.  Kernel times are averages of back-to-back launches between two HIP
events on the stream the kernel is launched on.  `roofline` is for the
dominant kernel (the fused prefill attention of the headline workload);
`traffic` comes from the rocprofv3 FETCH_SIZE / WRITE_SIZE summary in
profiles/ when that summary was taken on the current kernel source, else
null.  `cpu_baseline` times the CPU oracle (test infrastructure) on a bounded
sample of the same workload.

    python bench.py --profile {gemma2,qwen3,llama,decode} [--steps K]

runs only that workload's step (K launches after settling), for profiler
runs, and prints one short JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MXFP4_PEAK_TFLOPS = 10066.0   # MI355X dense FP4 (spec)
BF16_PEAK_TFLOPS = 2500.0
HBM_PEAK_GBS = 8000.0
METRIC = "attention TFLOPS (prefill) and HBM GB/s (decode) vs MI355X MXFP4 roofline"
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "attn_prefill_mxfp4_gemma2_9b_traffic.md")
KERNEL_SRC = os.path.join(ROOT, "bit_flashattention_hifa4_amd", "csrc", "attn_mxfp4.hip")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def read_traffic():
    """HBM bytes per prefill launch from the committed rocprofv3 counter summary, if current."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    text = open(TRAFFIC_SUMMARY).read()
    m_sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != kernel_source_sha():
        return None
    return float(m_b.group(1))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def settle(fn, torch, min_ms=200.0):
    """Run fn untimed until the GPU has been busy for min_ms.  MI355X raises its
    clocks over the first few tens of ms of sustained load (measured: a launch
    takes ~15% longer in the first 10 ms than after 35 ms), so a short warm-up
    alone would time the ramp instead of the sustained rate."""
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def copy_calibration(torch, dev, nbytes=256 << 20, reps=3):
    """A plain device copy of known size (nbytes read, nbytes written), for scaling the
    profiler's FETCH_SIZE / WRITE_SIZE counters; run only with --copy-calibration."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("copy calibration: %d x %d bytes" % (reps, nbytes))


def time_batch(fn, n, torch):
    """Average ms of n back-to-back launches of fn between two HIP events on the
    current stream (the per-launch form adds each event's own gap)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


class Prefill:
    """Device inputs and the step of one prefill workload."""

    def __init__(self, W, hb, torch, cfg, dev, tau):
        self.cfg, self.hb, self.tau = cfg, hb, tau
        log("generating", cfg.name)
        self.inp = W.prefill_inputs(cfg)
        self.q, self.k, self.v = (self.inp[n].to(dev) for n in ("q", "k", "v"))
        sm = self.inp["smooth"]
        self.smooth = torch.from_numpy(sm).to(dev) if sm is not None else None
        self.mx = hb.alloc_mx(cfg.B, cfg.Hq, cfg.Hkv, cfg.S, cfg.S, cfg.d, device=dev)
        self.out = torch.empty((cfg.B, cfg.Hq, cfg.S, cfg.d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((cfg.B, cfg.Hq, cfg.S), dtype=torch.float32, device=dev)
        self.flops = cfg.flops()
        # HBM bytes of the quantise launch: bf16 K, V in; codes + scales out; s
        self.q_bytes = (cfg.B * 2 * cfg.Hkv * cfg.S * cfg.d) * (2 + 17 / 32) + cfg.Hkv * cfg.d * 4

    # The step: Smooth-QK + MXFP4 of K and V (one launch), then the attention
    # kernel, which smooths and quantises its own Q rows in its prologue.
    def quantise(self, rule=None):
        self.hb.hifa4_quantize_qkv(None, self.k, self.v, self.smooth, out=self.mx,
                                   scale_rule=self.hb.SCALE_OCP if rule is None else rule)

    def attend(self, tau=None, normaliser=0, rule=0):
        self.hb.hifa4_attn_fwd_qraw(self.q, self.smooth, self.mx, causal=self.cfg.causal,
                                    out=self.out, lse=self.lse,
                                    rescale_threshold=self.tau if tau is None else tau,
                                    normaliser=normaliser, scale_rule=rule)

    def step(self):
        self.quantise()
        self.attend()

    def quantise_qkv(self):
        self.hb.hifa4_quantize_qkv(self.q, self.k, self.v, self.smooth, out=self.mx)

    def attend_codes(self):
        self.hb.hifa4_attn_fwd(self.mx, causal=self.cfg.causal, out=self.out, lse=self.lse,
                               rescale_threshold=self.tau)


def time_step(P, args, torch):
    """K steps back to back: wall ms and GPU ms per step."""
    settle(P.step, torch)
    for _ in range(args.warmup):
        P.step()
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    t_start.record()
    for _ in range(args.steps):
        P.step()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / args.steps, t_start.elapsed_time(t_end) / args.steps


def mfma_rate(torch, dev):
    """FP4 rate of a pure-MFMA kernel (the probe library's: four independent chains of
    32x32x64 FP4 MFMAs per wave, two workgroups of four waves per compute unit): the
    matrix-core ceiling a kernel reaches on this machine, next to the 10.066 PF figure."""
    import ctypes
    from bit_flashattention_hifa4_amd import build
    lib = ctypes.CDLL(build.PROBES_LIB)
    lib.probe_mfma_rate.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    blocks, iters = 512 * 8, 2000
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    f = lambda: lib.probe_mfma_rate(out.data_ptr(), blocks, iters, s)
    settle(f, torch, 100.0)
    ms = time_batch(f, 5, torch)
    flops = blocks * 4 * iters * 4 * 2.0 * 32 * 32 * 64
    return flops / (ms * 1e-3) / 1e12


def evented_quantise(P, n, torch):
    """Average ms of the step's quantise launch, from events recorded around it inside n
    back-to-back steps.  Launched back to back on its own, a quantise of a few
    microseconds is bound by the host's launch rate (measured: 24.9 us per launch for a
    6.2 us kernel); between attention launches the host stays ahead of the GPU."""
    settle(P.step, torch, 50.0)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for e0, e1 in ev:
        e0.record()
        P.quantise()
        e1.record()
        P.attend()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / n


def prefill_leg(P, args, torch, mfma_tflops):
    """Step and attention times of one prefill workload, with the attention's rate against
    the FP4 peak and against the measured pure-MFMA rate."""
    ms_wall, ms_gpu = time_step(P, args, torch)
    settle(P.attend, torch, 50.0)
    attn = time_batch(P.attend, args.steps, torch)
    quant = evented_quantise(P, args.steps, torch)
    tf = P.flops / (attn * 1e-3) / 1e12
    res = {"step_ms": ms_wall, "step_gpu_ms": ms_gpu, "attention_us": attn * 1e3,
           "attention_tflops": tf, "attention_fraction_of_fp4_peak": tf / MXFP4_PEAK_TFLOPS,
           "attention_fraction_of_measured_mfma_rate": tf / mfma_tflops if mfma_tflops else None,
           "quantize_kv_us": quant * 1e3,
           "quantize_kv_timing": "events around each launch inside back-to-back steps",
           "quantize_kv_gbs": P.q_bytes / (quant * 1e-3) / 1e9,
           "step_tflops": P.flops / (ms_wall * 1e-3) / 1e12, "flops": P.flops}
    log("%s: step %.1f us, attention %.1f us = %.1f TFLOP/s (%.1f%% of FP4 peak, %.1f%% of the "
        "measured MFMA rate), quantise K, V %.1f us"
        % (P.cfg.name, ms_wall * 1e3, attn * 1e3, tf, 100 * tf / MXFP4_PEAK_TFLOPS,
           100 * tf / mfma_tflops if mfma_tflops else float("nan"), quant * 1e3))
    return res


def variants_leg(P, args, torch, W):
    """The headline attention in other configurations: unfused step, threshold 0, the
    pages' non-reordered normaliser, the no-clip scale rule, RoPE in the quantise launch."""
    hb = P.hb
    res = {}
    n = max(5, args.steps // 2)

    def unfused():
        P.quantise_qkv()
        P.attend_codes()
    settle(unfused, torch, 50.0)
    res["unfused_step_ms"] = time_batch(unfused, n, torch)
    settle(P.attend_codes, torch, 50.0)
    res["unfused_attention_on_q_codes_us"] = time_batch(P.attend_codes, n, torch) * 1e3
    P.quantise()

    f0 = lambda: P.attend(tau=0.0)
    settle(f0, torch, 50.0)
    t0 = time_batch(f0, n, torch)
    res["attention_tau0_us"] = t0 * 1e3
    res["attention_tau0_tflops"] = P.flops / (t0 * 1e-3) / 1e12

    fd = lambda: P.attend(normaliser=hb.NORMALISER_DIRECT)
    settle(fd, torch, 50.0)
    td = time_batch(fd, n, torch)
    res["attention_direct_normaliser_us"] = td * 1e3

    def step_noclip():
        P.quantise(rule=hb.SCALE_NOCLIP)
        P.attend(rule=hb.SCALE_NOCLIP)
    settle(step_noclip, torch, 50.0)
    res["step_noclip_ms"] = time_batch(step_noclip, n, torch)
    P.quantise()

    cfg = P.cfg
    theta = cfg.rope_theta or 1.0e4
    cos, sin = (torch.from_numpy(t).to(P.q.device) for t in W.rope_tables(cfg.S, cfg.d, theta))

    def step_rope():
        hb.hifa4_quantize_qkv_rope(None, P.k, P.v, cos, sin, smooth=P.smooth, out=P.mx,
                                   Hkv=cfg.Hkv)
        P.attend()
    settle(step_rope, torch, 50.0)
    res["step_rope_kv_ms"] = time_batch(step_rope, n, torch)
    P.quantise()
    log("variants: unfused step %.1f us, tau 0 %.1f us, direct normaliser %.1f us, no-clip "
        "step %.1f us, RoPE step %.1f us" % (res["unfused_step_ms"] * 1e3,
                                             res["attention_tau0_us"],
                                             res["attention_direct_normaliser_us"],
                                             res["step_noclip_ms"] * 1e3,
                                             res["step_rope_kv_ms"] * 1e3))
    return res


def bf16_leg(P, args, torch):
    hb = P.hb
    bout = torch.empty_like(P.out)
    blse = torch.empty_like(P.lse)
    f = lambda: hb.bf16_attn_fwd(P.q, P.k, P.v, causal=P.cfg.causal, out=bout, lse=blse,
                                 rescale_threshold=P.tau)
    settle(f, torch)
    ms = time_batch(f, max(5, args.steps // 2), torch)
    tf = P.flops / (ms * 1e-3) / 1e12
    return ms, tf


def context_leg(hb, torch, dev, tau):
    """The prefill attention kernel (Q quantised in its prologue) on the Qwen3 head shape
    (32 query / 8 KV heads, d 128, causal, B 1) at 8k, 16k and 32k tokens: a 128-row
    item then runs up to 128, 256 and 512 key tiles instead of 64, so its fixed costs
    weigh less.  Inputs: N(0, 1) bf16 drawn on the GPU (torch generator, seed 0), no
    smoothing; settled clocks; back-to-back launches."""
    res = {}
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    B, Hq, Hkv, d = 1, 32, 8, 128
    for S in (8192, 16384, 32768):
        q = torch.randn(B, Hq, S, d, device=dev, generator=g).to(torch.bfloat16)
        k = torch.randn(B, Hkv, S, d, device=dev, generator=g).to(torch.bfloat16)
        v = torch.randn(B, Hkv, S, d, device=dev, generator=g).to(torch.bfloat16)
        mx = hb.hifa4_quantize_qkv(None, k, v, None, Hkv=Hkv)
        mx.Sq, mx.Hq = S, Hq
        out = torch.empty(B, Hq, S, d, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(B, Hq, S, dtype=torch.float32, device=dev)
        f = lambda: hb.hifa4_attn_fwd_qraw(q, None, mx, causal=True, out=out, lse=lse,
                                           rescale_threshold=tau)
        settle(f, torch)
        ms = time_batch(f, max(5, 81920 // S), torch)
        tflops = 4.0 * d * B * Hq * S * (S + 1) / 2 / (ms * 1e-3) / 1e12
        res["context_%dk_attention_ms" % (S // 1024)] = ms
        res["context_%dk_attention_tflops" % (S // 1024)] = tflops
        log("long-context prefill attention, S %d: %.3f ms, %.1f TFLOP/s (%.1f%% of FP4 peak)"
            % (S, ms, tflops, 100.0 * tflops / MXFP4_PEAK_TFLOPS))
        del q, k, v, mx, out, lse
    return res


def read_ceiling(torch, dev, nbytes=2 << 30):
    """HBM read rate of a plain streaming kernel (the probe library's) over a
    buffer 8x the last-level cache: the practical ceiling next to the decode's
    rate, which the 8 TB/s peak is not."""
    import ctypes
    from bit_flashattention_hifa4_amd import build
    lib = ctypes.CDLL(build.PROBES_LIB)
    lib.probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_void_p]
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    best = 0.0
    for blocks in (1024, 2048, 8192):
        out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
        s = torch.cuda.current_stream().cuda_stream
        f = lambda: lib.probe_stream_read(buf.data_ptr(), nbytes, out.data_ptr(), blocks, s)
        for _ in range(3):
            f()
        ms = time_batch(f, 10, torch)
        best = max(best, nbytes / (ms * 1e-3) / 1e9)
    del buf
    log("plain streaming read over 2 GiB: %.1f GB/s" % best)
    return {"stream_read_ceiling_gbs": best}


class Decode:
    """The 64-sequence MXFP4 cache, in `copies` copies so that repeated launches cannot be
    served by the 256 MB last-level cache (each copy is 1.2 GB)."""

    def __init__(self, W, hb, torch, np, dev, copies):
        cfg = self.cfg = W.DECODE
        self.hb, self.torch = hb, torch
        lens = self.lens = W.decode_lengths(cfg)
        cap = self.cap = int(-(-(int(lens.max()) + 1) // 64) * 64)  # room for one new token
        log("building the decode cache: %d sequences, %d tokens" % (cfg.B, int(lens.sum())))
        mx = hb.alloc_mx(cfg.B, cfg.Hq, cfg.Hkv, 1, cap, cfg.d, device=dev)
        hb.hifa4_quantize_qkv(W.decode_q(cfg).to(dev), None, None, None, out=mx)
        for b, L in enumerate(lens):
            kk, vv = W.decode_kv(cfg, b, int(L))
            sl = hb.MXQKV(None, None, mx.k_codes[b:b + 1], mx.k_scales[b:b + 1],
                          mx.v_codes[b:b + 1], mx.v_scales[b:b + 1], 1, cfg.Hq, cfg.Hkv, 0,
                          int(L), cfg.d, cap)
            hb.hifa4_quantize_qkv(None, kk.to(dev), vv.to(dev), None, kv_stride=cap, out=sl)
        mx.Sq, mx.Sk, mx.kv_stride = 1, cap, cap
        self.mxs = [mx]
        for _ in range(copies - 1):
            c = hb.MXQKV(mx.q_codes, mx.q_scales, mx.k_codes.clone(), mx.k_scales.clone(),
                         mx.v_codes.clone(), mx.v_scales.clone(), mx.B, mx.Hq, mx.Hkv, 1, cap,
                         mx.d, cap)
            self.mxs.append(c)
        self.lens_t = torch.from_numpy(lens.astype(np.int32)).to(dev)
        self.out = torch.empty((cfg.B, cfg.Hq, 1, cfg.d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((cfg.B, cfg.Hq, 1), dtype=torch.float32, device=dev)
        p = hb.make_params(cfg.B, cfg.Hq, cfg.Hkv, 1, cap, cfg.d, causal=True, kv_stride=cap,
                           kv_lens=self.lens_t)
        self.ws = torch.empty(hb.hifa4_attn_workspace_size(p), dtype=torch.uint8, device=dev)
        self.i = 0
        L = lens.astype(np.int64)
        # algorithmic bytes: valid-token K (codes + scales), V blocks covering the valid
        # tokens, bf16 Q and O
        kv = cfg.Hkv * (L * (cfg.d // 2 + cfg.d // 32)).sum() \
            + cfg.Hkv * (((L + 31) // 32) * 32 * (cfg.d // 2 + cfg.d // 32)).sum()
        self.bytes = float(kv + 2 * cfg.B * cfg.Hq * cfg.d * 2)

    def attend(self):
        mx = self.mxs[self.i]
        self.i = (self.i + 1) % len(self.mxs)
        self.hb.hifa4_attn_fwd(mx, causal=True, kv_lens=self.lens_t, out=self.out, lse=self.lse,
                               workspace=self.ws,
                               rescale_threshold=self.hb.RESCALE_THRESHOLD_FAST)


def decode_leg(W, hb, torch, np, dev, args):
    D = Decode(W, hb, torch, np, dev, copies=3)
    cfg = D.cfg
    settle(D.attend, torch)
    ms = time_batch(D.attend, max(12, args.steps), torch)
    gbs = D.bytes / (ms * 1e-3) / 1e9
    log("decode %.3f ms over 3 rotating cache copies: %.1f GB/s (%.1f%% of HBM peak)"
        % (ms, gbs, gbs / HBM_PEAK_GBS * 100))
    res = {"decode_workload": cfg.name, "decode_tokens": int(D.lens.sum()),
           "decode_ms_avg": ms, "decode_bytes": D.bytes, "decode_gbs": gbs,
           "decode_fraction_of_hbm_peak": gbs / HBM_PEAK_GBS,
           "decode_timing": "back-to-back launches rotating over 3 copies of the 1.2 GB cache"}

    # the whole decode step: append one token per sequence (RoPE at its position,
    # K row, value-block requantisation, new Q) then attention over L + 1 keys.
    # Repeating it rewrites the same rows from the same lengths, so every
    # repetition does the same work.
    mx = D.mxs[0]
    rng = np.random.default_rng(cfg.seed + 5)
    new = [torch.from_numpy(rng.standard_normal((cfg.B, h, 1, cfg.d), dtype=np.float32))
           .to(torch.bfloat16).to(dev) for h in (cfg.Hq, cfg.Hkv, cfg.Hkv)]
    cos, sin = (torch.from_numpy(t).to(dev) for t in W.rope_tables(D.cap, cfg.d, 1.0e6))
    tail = hb.alloc_v_tail(cfg.B, cfg.Hkv, cfg.d, device=dev)
    lens_new = torch.empty_like(D.lens_t)

    def append():
        hb.hifa4_kv_append(new[0], new[1], new[2], D.lens_t, mx, tail, kv_lens_out=lens_new,
                           cos=cos, sin=sin)

    def attend_new():
        hb.hifa4_attn_fwd(mx, causal=True, kv_lens=lens_new, out=D.out, lse=D.lse,
                          workspace=D.ws, rescale_threshold=hb.RESCALE_THRESHOLD_FAST)

    def dstep():
        append()
        attend_new()

    settle(dstep, torch)
    n = max(10, args.steps)
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(n)]
    for e0, e1, e2 in evs:
        e0.record()
        append()
        e1.record()
        attend_new()
        e2.record()
    torch.cuda.synchronize()
    ap_ms = np.array([a.elapsed_time(b) for a, b, _ in evs])
    st_ms = np.array([a.elapsed_time(c) for a, _, c in evs])
    log("decode step %.3f ms (append %.3f ms + attention over L + 1)" % (st_ms.mean(), ap_ms.mean()))
    res.update({"decode_step_definition": "hifa4_kv_append (1 token: RoPE, K row, V block "
                                          "requantisation, Q) + hifa4_attn_fwd over L + 1 keys",
                "decode_step_ms_avg": float(st_ms.mean()),
                "decode_append_ms_avg": float(ap_ms.mean())})
    del D
    return res


def cpu_baseline(W, P, np, torch):
    """The CPU oracle on a bounded sample of the headline workload: batch entry 0, every
    head (a quarter of the Gemma2-shaped batch).  Times the oracle's MXFP4 quantisation of
    the sample + its P-Reordering attention (the `value`), and its exact mode (no
    quantisation) on the same rows; from the same runs, the accuracy of the GPU output on
    the sample (against exact fp64 attention and against the oracle, in units of max|V|)
    and the oracle's per-tile normaliser-mismatch statistic of the non-reordered form."""
    import oracle

    cfg = P.cfg
    qs = W.to_f32(P.inp["q"][:1])
    ks = W.to_f32(P.inp["k"][:1])
    vs = W.to_f32(P.inp["v"][:1])
    nthreads = oracle.default_threads()
    t0 = time.perf_counter()
    qq = oracle.quantize_qkv(qs, ks, vs, P.inp["smooth"])
    r = oracle.attention(qq["q_deq"], qq["k_deq"], qq["v_deq"], causal=cfg.causal, bc=64,
                         quant_p=True, nthreads=nthreads, tau=P.tau, want_eps=True)
    dt = time.perf_counter() - t0
    t1 = time.perf_counter()
    ex = oracle.attention(qs, ks, vs, causal=cfg.causal, bc=64, quant_p=False, nthreads=nthreads)
    dt_exact = time.perf_counter() - t1
    pairs = cfg.S * (cfg.S + 1) // 2 if cfg.causal else cfg.S * cfg.S
    flops = 4.0 * cfg.d * pairs * cfg.Hq
    # the GPU output of the same rows: the step's attention on the step's inputs
    P.step()
    torch.cuda.synchronize()
    o = P.out[:1].float().cpu().numpy()
    vmax = float(np.abs(vs).max())
    e_ex = o - ex["o"]
    e_or = o - r["o"]
    eps = r["eps_tile_mean"]
    eps = eps[np.isfinite(eps)]
    acc = {"sample": "batch entry 0, all %d query heads, all %d rows" % (cfg.Hq, cfg.S),
           "max_abs_err_vs_exact_over_max_abs_v": float(np.abs(e_ex).max() / vmax),
           "rms_err_vs_exact_over_max_abs_v": float(np.sqrt(np.mean(e_ex ** 2)) / vmax),
           "max_abs_err_vs_oracle_over_max_abs_v": float(np.abs(e_or).max() / vmax),
           "rms_err_vs_oracle_over_max_abs_v": float(np.sqrt(np.mean(e_or ** 2)) / vmax),
           "gate_max_abs_over_max_abs_v": 2e-2,
           "eps_bar_tiles": int(eps.size),
           "eps_bar_tile": "128 query rows x 64 keys, rescale threshold %g" % P.tau,
           "eps_bar_median": float(np.median(eps)),
           "eps_bar_fraction_negative": float((eps < 0).mean())}
    log("accuracy on the sample: max|O - exact| = %.4g, rms %.4g; max|O - oracle| = %.4g "
        "(x max|V|); eps_bar median %.4f, %.1f%% of %d tiles negative"
        % (acc["max_abs_err_vs_exact_over_max_abs_v"], acc["rms_err_vs_exact_over_max_abs_v"],
           acc["max_abs_err_vs_oracle_over_max_abs_v"], acc["eps_bar_median"],
           100 * acc["eps_bar_fraction_negative"], eps.size))
    base = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "%s, batch entry 0 of %d (all %d query heads): MXFP4 quantisation of the "
                      "sample + online-softmax attention with P-Reordering, fp64, %.1f s on %d "
                      "threads" % (cfg.name, cfg.B, cfg.Hq, dt, nthreads),
            "oracle_exact_mode_s": dt_exact,
            "oracle_exact_mode_tflops": flops / dt_exact / 1e12}
    return base, acc


def profile_main(args, W, hb, torch, np, dev):
    """Only the named workload's step, for profiler runs (rocprofv3)."""
    tau = hb.RESCALE_THRESHOLD_FAST
    if args.profile == "decode":
        D = Decode(W, hb, torch, np, dev, copies=3)
        settle(D.attend, torch, 50.0)
        ms = time_batch(D.attend, args.steps, torch)
        if args.copy_calibration:
            copy_calibration(torch, dev)
        print(json.dumps({"profile": "decode", "decode_ms_avg": ms,
                          "decode_gbs": D.bytes / (ms * 1e-3) / 1e9,
                          "decode_bytes": D.bytes}), flush=True)
        return
    cfg = {"gemma2": W.GEMMA2_9B, "qwen3": W.QWEN3_8B, "llama": W.LLAMA31_8B}[args.profile]
    P = Prefill(W, hb, torch, cfg, dev, tau)
    settle(P.step, torch, 50.0)
    ms = time_batch(P.step, args.steps, torch)
    if args.copy_calibration:
        copy_calibration(torch, dev)
    print(json.dumps({"profile": cfg.name, "step_ms": ms, "flops": P.flops,
                      "kernel_source_sha256_16": kernel_source_sha()}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-bf16", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the long-context prefill attention leg")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the headline's variants (unfused, threshold 0, direct "
                         "normaliser, no-clip rule, RoPE in the quantise launch)")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the Qwen3- and Llama-shaped prefill legs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 256 MiB device copy (for profiler byte-counter scaling)")
    ap.add_argument("--profile", choices=["gemma2", "qwen3", "llama", "decode"],
                    help="run only that workload's step, for profiler runs")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the attention path runs on one GPU only (it has no multi-GPU "
              "leg); got --gpus %d, WORLD_SIZE %d" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from bit_flashattention_hifa4_amd import binding as hb
    from bit_flashattention_hifa4_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    hb.load_library()
    dev = torch.device("cuda:0")
    if args.profile:
        profile_main(args, W, hb, torch, np, dev)
        return
    tau = hb.RESCALE_THRESHOLD_FAST
    mfma_tf = mfma_rate(torch, dev)
    log("pure FP4 MFMA rate: %.0f TFLOP/s (%.1f%% of the 10.066 PF figure)"
        % (mfma_tf, 100 * mfma_tf / MXFP4_PEAK_TFLOPS))

    # ---- headline: the Gemma2-9B-shaped prefill step
    P = Prefill(W, hb, torch, W.GEMMA2_9B, dev, tau)
    cfg = P.cfg
    ms_per_step, gpu_ms_per_step = time_step(P, args, torch)
    value = P.flops / (ms_per_step * 1e-3) / 1e12

    # per-kernel split of the step (events around each launch)
    settle(P.step, torch, 50.0)
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
          for _ in range(args.steps)]
    for e0, e1, e2 in ev:
        e0.record()
        P.quantise()
        e1.record()
        P.attend()
        e2.record()
    torch.cuda.synchronize()
    q_ms = np.array([a.elapsed_time(b) for a, b, _ in ev])
    a_ms = np.array([b.elapsed_time(c) for _, b, c in ev])
    # the roofline's launch duration: the step's attention launched back to back
    settle(P.attend, torch, 50.0)
    attn_avg = time_batch(P.attend, args.steps, torch)
    achieved = P.flops / (attn_avg * 1e-3) / 1e12
    log("headline %s: step %.1f us wall, %.1f us GPU (quantise %.1f us, attention %.1f us): "
        "%.1f TFLOP/s step, %.1f attention (%.1f%% of FP4 peak)"
        % (cfg.name, ms_per_step * 1e3, gpu_ms_per_step * 1e3, q_ms.mean() * 1e3,
           attn_avg * 1e3, value, achieved, 100 * achieved / MXFP4_PEAK_TFLOPS))

    extra = {
        "step_definition": "hifa4_quantize_qkv(K, V) + hifa4_attn_fwd_qraw (Q smoothed and "
                           "quantised in the attention prologue)",
        "step_gpu_ms": gpu_ms_per_step,
        "attention_us": attn_avg * 1e3,
        "attention_timing": "K back-to-back launches between two HIP events on the launch "
                            "stream; the evented step pass (events around each launch) below",
        "attention_evented_us_p10_p50_p90": [float(np.percentile(a_ms, p)) * 1e3
                                             for p in (10, 50, 90)],
        "attention_tflops": achieved,
        "attention_fraction_of_measured_mfma_rate": achieved / mfma_tf,
        "quantize_kv_us": float(q_ms.mean()) * 1e3,
        "quantize_kv_gbs": P.q_bytes / (q_ms.mean() * 1e-3) / 1e9,
        "flops_per_step": P.flops,
        "mfma_fp4_measured_tflops": mfma_tf,
        # the clock at which a full-rate FP4 MFMA stream gives the measured rate (the
        # probe issues independent chains only): the headline fraction against the
        # observed clock is attention_fraction_of_measured_mfma_rate
        "clock_implied_by_mfma_probe_ghz": 2.4 * mfma_tf / MXFP4_PEAK_TFLOPS,
        "kernel_source_sha256_16": kernel_source_sha(),
    }
    if not args.no_variants:
        extra["variants"] = variants_leg(P, args, torch, W)
    if not args.no_bf16:
        b_ms, b_tf = bf16_leg(P, args, torch)
        extra["bf16_attention_us"] = b_ms * 1e3
        extra["bf16_attention_tflops"] = b_tf
        extra["bf16_fraction_of_bf16_peak"] = b_tf / BF16_PEAK_TFLOPS
        extra["mxfp4_over_bf16_latency_ratio"] = attn_avg / b_ms
        log("bf16 baseline %.1f us (%.1f TFLOP/s, %.1f%% of bf16 peak); MXFP4 / bf16 latency "
            "%.3f" % (b_ms * 1e3, b_tf, 100 * b_tf / BF16_PEAK_TFLOPS, attn_avg / b_ms))

    cpu = acc = None
    if not args.no_cpu:
        log("timing the CPU oracle on a sample")
        cpu, acc = cpu_baseline(W, P, np, torch)
        extra["accuracy"] = acc
    del P
    torch.cuda.empty_cache()

    # ---- the other prefill configurations, each timed the same way
    if not args.no_legs:
        legs = {}
        for c in (W.QWEN3_8B, W.LLAMA31_8B):
            Pc = Prefill(W, hb, torch, c, dev, tau)
            legs[c.name] = prefill_leg(Pc, args, torch, mfma_tf)
            if c is W.QWEN3_8B and not args.no_bf16:
                b_ms, b_tf = bf16_leg(Pc, args, torch)
                legs[c.name]["bf16_attention_us"] = b_ms * 1e3
                legs[c.name]["bf16_fraction_of_bf16_peak"] = b_tf / BF16_PEAK_TFLOPS
                legs[c.name]["mxfp4_over_bf16_latency_ratio"] = \
                    legs[c.name]["attention_us"] / (b_ms * 1e3)
                log("%s bf16 baseline %.1f us (%.1f%% of bf16 peak)"
                    % (c.name, b_ms * 1e3, 100 * b_tf / BF16_PEAK_TFLOPS))
            del Pc
            torch.cuda.empty_cache()
        extra["prefill_legs"] = legs

    if not args.no_decode:
        extra.update(decode_leg(W, hb, torch, np, dev, args))
        torch.cuda.empty_cache()
    if not args.no_context:
        extra.update(context_leg(hb, torch, dev, tau))
    if args.copy_calibration:
        copy_calibration(torch, dev)
    if not args.no_decode:
        extra.update(read_ceiling(torch, dev))

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv,
                   "S": cfg.S, "d": cfg.d, "causal": cfg.causal, "rescale_threshold": tau,
                   "step": "hifa4_quantize_qkv(K, V) + hifa4_attn_fwd_qraw",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MXFP4_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MXFP4_PEAK_TFLOPS,
                     "traffic": read_traffic()},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
