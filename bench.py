#!/usr/bin/env python3
"""Benchmark of the MXFP4 FlashAttention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline workload: the Qwen3-8B-shaped causal prefill layer (B=1, 32 query
heads, 8 KV heads, d=128, S=4096, bf16 inputs after synthetic RoPE, 4 outlier
key channels per head, calibration-static smoothing).  One step is one pass of
the whole hot path over that batch, inputs resident in HBM: Smooth-QK + MXFP4
quantisation of K and V (one launch), then the fused MXFP4 attention, which
smooths and quantises its own Q rows in its prologue (one launch; the codes
are bit-identical to quantising Q separately).  `value` = algorithmic
attention flops (4 d per unmasked query-key pair) per second of step time.

The attention runs with the lazy-rescale threshold 8 (log2 units; the running
max moves only when a tile's max exceeds it by more than that, and P_hat is
defined in that frame; the CPU oracle takes the same value).

Also reported (in "extra"): the step's kernels one by one, the unfused step
(Q, K, V quantised in one launch, attention on Q codes), the step with RoPE of
pre-rotation K inside the quantise launch, the attention with threshold 0 (the
FlashAttention-2 frame) and with the pages' non-reordered normaliser, the step
under the no-clip block-scale rule (a format variant), the bf16
FlashAttention baseline on the same prefill (time ratio = the measured
counterpart of the pages' projected latency cut), the same attention kernel at
8k-32k tokens (long-context prefill), the split-K decode on 64
sequences with 1k-32k MXFP4 cache entries (HBM GB/s, split + merge), the
decode step (one-token cache append + attention), and the HBM read rate of a
plain streaming kernel on the same box.

Every timed region follows at least 200 ms of untimed launches of the same
work (the GPU's clocks ramp up under sustained load), then the W warm-up
steps.  Kernel times are averages of back-to-back launches between two HIP
events on the stream the kernel is launched on (events around every launch
add their own gaps; that evented pass is reported separately).  `roofline` is
for the dominant kernel (the fused prefill attention); `traffic` comes from
the rocprofv3 FETCH_SIZE / WRITE_SIZE summary in profiles/ when that summary
was taken on the current kernel source, else null.  `cpu_baseline` times the
CPU oracle (test infrastructure) on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MXFP4_PEAK_TFLOPS = 10066.0   # MI355X dense FP4 (spec)
BF16_PEAK_TFLOPS = 2500.0
HBM_PEAK_GBS = 8000.0
METRIC = "attention TFLOPS (prefill) and HBM GB/s (decode) vs MI355X MXFP4 roofline"
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "attn_prefill_mxfp4_qwen3_8b_traffic.md")
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


def cpu_baseline(W, cfg, inp, n_kv_heads=None):
    """The CPU oracle on a bounded sample of the prefill workload: its first n_kv_heads KV
    heads with their query heads (all of them by default, i.e. the whole batch: about 7 s
    on 16 cores).  Includes the oracle's quantisation of the sample.
    """
    import oracle

    g = cfg.Hq // cfg.Hkv
    nk = cfg.Hkv if n_kv_heads is None else n_kv_heads
    heads = list(range(nk * g))
    qs = W.to_f32(inp["q"][:, :nk * g])
    ks = W.to_f32(inp["k"][:, :nk])
    vs = W.to_f32(inp["v"][:, :nk])
    sm = inp["smooth"][:nk] if inp["smooth"] is not None else None
    nthreads = oracle.default_threads()
    t0 = time.perf_counter()
    qq = oracle.quantize_qkv(qs, ks, vs, sm)
    oracle.attention(qq["q_deq"], qq["k_deq"], qq["v_deq"], causal=cfg.causal, bc=64,
                     quant_p=True, nthreads=nthreads)
    dt = time.perf_counter() - t0
    pairs = cfg.S * (cfg.S + 1) // 2 if cfg.causal else cfg.S * cfg.S
    flops = 4.0 * cfg.d * pairs * len(heads) * cfg.B
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
            "sample": "%s, %d of %d query heads (KV heads 0..%d): MXFP4 quantisation of the "
                      "sample + online-softmax attention with P-Reordering, fp64, %.1f s on %d "
                      "threads" % (cfg.name, len(heads), cfg.Hq, nk - 1, dt, nthreads)}


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
    ap.add_argument("--no-unfused", action="store_true",
                    help="skip the step variant with Q quantised by the quantise kernel")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 256 MiB device copy (for profiler byte-counter scaling)")
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
    cfg = W.QWEN3_8B
    log("generating", cfg.name)
    inp = W.prefill_inputs(cfg)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    smooth = torch.from_numpy(inp["smooth"]).to(dev)
    mx = hb.alloc_mx(cfg.B, cfg.Hq, cfg.Hkv, cfg.S, cfg.S, cfg.d, device=dev)
    out = torch.empty((cfg.B, cfg.Hq, cfg.S, cfg.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((cfg.B, cfg.Hq, cfg.S), dtype=torch.float32, device=dev)
    flops = cfg.flops()
    tau = hb.RESCALE_THRESHOLD_FAST

    # The step: Smooth-QK + MXFP4 of K and V (one launch), then the attention
    # kernel, which smooths and quantises its own Q rows in its prologue (the
    # codes are bit-identical to quantising Q separately).
    def quantise():
        hb.hifa4_quantize_qkv(None, k, v, smooth, out=mx, scale_rule=hb.SCALE_OCP)

    def attend():
        hb.hifa4_attn_fwd_qraw(q, smooth, mx, causal=cfg.causal, out=out, lse=lse,
                               rescale_threshold=tau)

    def step():
        quantise()
        attend()

    # the same step with Q quantised by the quantise kernel (reported in extra)
    def quantise_qkv():
        hb.hifa4_quantize_qkv(q, k, v, smooth, out=mx)

    def attend_codes():
        hb.hifa4_attn_fwd(mx, causal=cfg.causal, out=out, lse=lse, rescale_threshold=tau)

    def step_unfused():
        quantise_qkv()
        attend_codes()

    # ---- headline: K timed steps of (quantise + attention), back to back
    settle(step, torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record()
    for _ in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    gpu_ms_per_step = t_start.elapsed_time(t_end) / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12

    # ---- per-kernel times: the same step with HIP events around each launch
    settle(step, torch, 50.0)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1, e2 in ev:
        e0.record()
        quantise()
        e1.record()
        attend()
        e2.record()
    torch.cuda.synchronize()
    q_ms = np.array([a.elapsed_time(b) for a, b, _ in ev])
    a_ms = np.array([b.elapsed_time(c) for _, b, c in ev])
    # the roofline's launch duration: the step's attention launched back to back
    # (inputs unchanged between launches), so the events add one gap per batch
    settle(attend, torch, 50.0)
    attn_avg = time_batch(attend, args.steps, torch)
    achieved = flops / (attn_avg * 1e-3) / 1e12
    q_bytes = (cfg.B * 2 * cfg.Hkv * cfg.S * cfg.d) * (2 + 17 / 32) + cfg.Hkv * cfg.d * 4
    log("step %.3f ms wall, %.3f ms GPU (quantise %.3f ms, attention %.3f ms): %.1f TFLOP/s step, "
        "%.1f attention" % (ms_per_step, gpu_ms_per_step, q_ms.mean(), attn_avg, value, achieved))

    # ---- the unfused step (Q quantised by the quantise kernel, read back as codes)
    unfused = {}
    if not args.no_unfused:
        settle(step_unfused, torch, 50.0)
        evu = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
                torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for e0, e1, e2 in evu:
            e0.record()
            quantise_qkv()
            e1.record()
            attend_codes()
            e2.record()
        torch.cuda.synchronize()
        uq_ms = np.array([a.elapsed_time(b) for a, b, _ in evu])
        ua_ms = np.array([b.elapsed_time(c) for _, b, c in evu])
        u_ms = np.array([a.elapsed_time(c) for a, _, c in evu])
        log("unfused step %.3f ms (quantise Q, K, V %.3f ms, attention on codes %.3f ms)"
            % (u_ms.mean(), uq_ms.mean(), ua_ms.mean()))
        unfused = {"unfused_step_ms_avg": float(u_ms.mean()),
                   "unfused_quantize_qkv_ms_avg": float(uq_ms.mean()),
                   "unfused_attention_ms_avg": float(ua_ms.mean())}

    extra = {
        "step_definition": "hifa4_quantize_qkv(K, V) + hifa4_attn_fwd_qraw (Q smoothed and "
                           "quantised in the attention prologue)",
        "step_gpu_ms": gpu_ms_per_step,
        "attention_ms_avg": attn_avg,
        "attention_timing": "K back-to-back launches between two HIP events on the launch "
                            "stream; the evented step pass (events around each launch) below",
        "attention_evented_ms_avg": float(a_ms.mean()),
        "attention_evented_ms_p10_p50_p90": [float(np.percentile(a_ms, p)) for p in (10, 50, 90)],
        "attention_tflops": achieved,
        "quantize_kv_ms_avg": float(q_ms.mean()),
        "quantize_kv_gbs": q_bytes / (q_ms.mean() * 1e-3) / 1e9,
        **unfused,
        "flops_per_step": flops,
        "kernel_source_sha256_16": kernel_source_sha(),
    }

    # ---- the step with RoPE of K in the quantise launch (the headline step takes
    #      post-RoPE activations; this one rotates pre-RoPE K in the same pass),
    #      timed back to back like the headline
    cos, sin = (torch.from_numpy(t).to(dev) for t in W.rope_tables(cfg.S, cfg.d, cfg.rope_theta))

    def step_rope():
        hb.hifa4_quantize_qkv_rope(None, k, v, cos, sin, smooth=smooth, out=mx, Hkv=cfg.Hkv)
        attend()

    settle(step_rope, torch, 50.0)
    n_r = max(5, args.steps // 2)
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record()
    for _ in range(n_r):
        step_rope()
    r1.record()
    torch.cuda.synchronize()
    extra["step_rope_kv_ms"] = r0.elapsed_time(r1) / n_r
    log("step with RoPE of K in the quantise launch: %.3f ms (headline step %.3f ms GPU)"
        % (extra["step_rope_kv_ms"], gpu_ms_per_step))
    quantise()   # restore the codes of the step's inputs

    # ---- the same attention in the FlashAttention-2 frame (rescale threshold 0)
    f0 = lambda: hb.hifa4_attn_fwd_qraw(q, smooth, mx, causal=cfg.causal, out=out, lse=lse,
                                        rescale_threshold=0.0)
    settle(f0, torch)
    z_ms = np.array([time_batch(f0, max(5, args.steps // 2), torch)])
    extra["attention_tau0_ms_avg"] = float(z_ms.mean())
    extra["attention_tau0_tflops"] = flops / (z_ms.mean() * 1e-3) / 1e12
    log("attention with rescale threshold 0: %.3f ms (%.1f TFLOP/s)"
        % (z_ms.mean(), extra["attention_tau0_tflops"]))

    # ---- the pages' ablation: the same attention with the non-reordered normaliser
    #      (l summed from the fp32 P on the vector ALU, no ones column)
    fd = lambda: hb.hifa4_attn_fwd_qraw(q, smooth, mx, causal=cfg.causal, out=out, lse=lse,
                                        rescale_threshold=tau, normaliser=hb.NORMALISER_DIRECT)
    settle(fd, torch)
    d_ms = np.array([time_batch(fd, max(5, args.steps // 2), torch)])
    extra["attention_direct_normaliser_ms_avg"] = float(d_ms.mean())
    extra["p_reordering_over_direct_latency_ratio"] = attn_avg / float(d_ms.mean())
    log("attention with the direct normaliser: %.3f ms (P-Reordering / direct latency %.3f)"
        % (d_ms.mean(), extra["p_reordering_over_direct_latency_ratio"]))

    # ---- the no-clip block-scale rule (a format variant): the same step with K and V
    #      quantised, Q quantised in the prologue and P_hat scaled under it
    def step_noclip():
        hb.hifa4_quantize_qkv(None, k, v, smooth, out=mx, scale_rule=hb.SCALE_NOCLIP)
        hb.hifa4_attn_fwd_qraw(q, smooth, mx, causal=cfg.causal, out=out, lse=lse,
                               rescale_threshold=tau, scale_rule=hb.SCALE_NOCLIP)
    settle(step_noclip, torch)
    extra["step_noclip_ms"] = float(time_batch(step_noclip, max(5, args.steps // 2), torch))
    log("step under the no-clip scale rule: %.3f ms (headline step %.3f ms GPU)"
        % (extra["step_noclip_ms"], gpu_ms_per_step))
    quantise()   # restore the step's codes

    # ---- bf16 FlashAttention baseline on the same inputs
    if not args.no_bf16:
        bout = torch.empty_like(out)
        blse = torch.empty_like(lse)
        f = lambda: hb.bf16_attn_fwd(q, k, v, causal=cfg.causal, out=bout, lse=blse,
                                     rescale_threshold=tau)
        settle(f, torch)
        b_ms = np.array([time_batch(f, max(5, args.steps // 2), torch)])
        extra["bf16_attention_ms_avg"] = float(b_ms.mean())
        extra["bf16_attention_tflops"] = flops / (b_ms.mean() * 1e-3) / 1e12
        extra["bf16_fraction_of_bf16_peak"] = extra["bf16_attention_tflops"] / BF16_PEAK_TFLOPS
        extra["mxfp4_over_bf16_latency_ratio"] = attn_avg / float(b_ms.mean())
        log("bf16 baseline %.3f ms (%.1f TFLOP/s); MXFP4 / bf16 latency %.3f"
            % (b_ms.mean(), extra["bf16_attention_tflops"], extra["mxfp4_over_bf16_latency_ratio"]))
        del bout, blse

    # ---- split-K decode against the long MXFP4 cache
    if not args.no_decode:
        extra.update(decode_leg(W, hb, torch, np, dev, args))
    if not args.no_context:
        extra.update(context_leg(hb, torch, dev, tau))

    if args.copy_calibration:
        copy_calibration(torch, dev)

    if not args.no_decode:
        extra.update(read_ceiling(torch, dev))

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle on a sample")
        cpu = cpu_baseline(W, cfg, inp)

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


def context_leg(hb, torch, dev, tau):
    """The step's attention kernel (Q quantised in its prologue) on the Qwen3-8B head
    shape (32 query / 8 KV heads, d 128, causal, B 1) at 8k, 16k and 32k tokens: a
    128-row item then runs up to 128, 256 and 512 key tiles instead of 64, so its
    fixed costs weigh less.  Inputs: N(0, 1) bf16 drawn on the GPU (torch generator,
    seed 0), no smoothing; settled clocks; back-to-back launches."""
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
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            f()
        e1.record()
        torch.cuda.synchronize()
        best = max(best, nbytes / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9)
    del buf
    log("plain streaming read over 2 GiB: %.1f GB/s" % best)
    return {"stream_read_ceiling_gbs": best}


def decode_leg(W, hb, torch, np, dev, args):
    cfg = W.DECODE
    lens = W.decode_lengths(cfg)
    cap = int(-(-(int(lens.max()) + 1) // 64) * 64)   # room for the decode step's new token
    log("building the decode cache: %d sequences, %d tokens" % (cfg.B, int(lens.sum())))
    mx = hb.alloc_mx(cfg.B, cfg.Hq, cfg.Hkv, 1, cap, cfg.d, device=dev)
    hb.hifa4_quantize_qkv(W.decode_q(cfg).to(dev), None, None, None, out=mx)
    for b, L in enumerate(lens):
        kk, vv = W.decode_kv(cfg, b, int(L))
        sl = hb.MXQKV(None, None, mx.k_codes[b:b + 1], mx.k_scales[b:b + 1], mx.v_codes[b:b + 1],
                      mx.v_scales[b:b + 1], 1, cfg.Hq, cfg.Hkv, 0, int(L), cfg.d, cap)
        hb.hifa4_quantize_qkv(None, kk.to(dev), vv.to(dev), None, kv_stride=cap, out=sl)
    mx.Sq, mx.Sk, mx.kv_stride = 1, cap, cap
    lens_t = torch.from_numpy(lens.astype(np.int32)).to(dev)
    out = torch.empty((cfg.B, cfg.Hq, 1, cfg.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((cfg.B, cfg.Hq, 1), dtype=torch.float32, device=dev)
    p = hb.make_params(cfg.B, cfg.Hq, cfg.Hkv, 1, cap, cfg.d, causal=True, kv_stride=cap,
                       kv_lens=lens_t)
    ws = torch.empty(hb.hifa4_attn_workspace_size(p), dtype=torch.uint8, device=dev)
    f = lambda: hb.hifa4_attn_fwd(mx, causal=True, kv_lens=lens_t, out=out, lse=lse, workspace=ws,
                                  rescale_threshold=hb.RESCALE_THRESHOLD_FAST)
    settle(f, torch)
    d_ms = np.array([time_batch(f, max(10, args.steps), torch)])
    # algorithmic bytes: valid-token K (codes + scales), V blocks covering the valid
    # tokens, bf16 Q and O
    L = lens.astype(np.int64)
    kv_bytes = cfg.Hkv * (L * (cfg.d // 2 + cfg.d // 32)).sum() \
        + cfg.Hkv * (((L + 31) // 32) * 32 * (cfg.d // 2 + cfg.d // 32)).sum()
    qo = 2 * cfg.B * cfg.Hq * cfg.d * 2
    total = float(kv_bytes + qo)
    gbs = total / (d_ms.mean() * 1e-3) / 1e9
    log("decode %.3f ms: %.1f GB/s (%.1f%% of HBM peak)" % (d_ms.mean(), gbs, gbs / HBM_PEAK_GBS * 100))
    res = {"decode_workload": cfg.name, "decode_tokens": int(lens.sum()),
           "decode_ms_avg": float(d_ms.mean()), "decode_bytes": total, "decode_gbs": gbs,
           "decode_fraction_of_hbm_peak": gbs / HBM_PEAK_GBS}

    # the whole decode step: append one token per sequence (RoPE at its position,
    # K row, value-block requantisation, new Q) then attention over L + 1 keys.
    # Repeating it rewrites the same rows from the same lengths, so every
    # repetition does the same work.
    rng = np.random.default_rng(cfg.seed + 5)
    new = [torch.from_numpy(rng.standard_normal((cfg.B, h, 1, cfg.d), dtype=np.float32))
           .to(torch.bfloat16).to(dev) for h in (cfg.Hq, cfg.Hkv, cfg.Hkv)]
    cos, sin = (torch.from_numpy(t).to(dev) for t in W.rope_tables(cap, cfg.d, 1.0e6))
    tail = hb.alloc_v_tail(cfg.B, cfg.Hkv, cfg.d, device=dev)
    lens_new = torch.empty_like(lens_t)

    def append():
        hb.hifa4_kv_append(new[0], new[1], new[2], lens_t, mx, tail, kv_lens_out=lens_new,
                           cos=cos, sin=sin)

    def attend_new():
        hb.hifa4_attn_fwd(mx, causal=True, kv_lens=lens_new, out=out, lse=lse, workspace=ws,
                          rescale_threshold=hb.RESCALE_THRESHOLD_FAST)

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
    return res


if __name__ == "__main__":
    main()
