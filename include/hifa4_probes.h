/*
 * hifa4_probes.h -- diagnostic entry points of libhifa4_probes.so.
 *
 * They run single gfx950 instructions on caller-supplied operands so that
 * tests can check, against host-side expectations, the facts the attention
 * kernels rely on: which lane holds which operand element and block scale of
 * the scaled-FP4 MFMA (the 4-bit products the HiFA4 abstract puts under both
 * Q K^T and P V), the accumulator layout, the rounding of the packed FP4
 * convert used to quantise P, and the issue rates of v_exp_f32 and the FP4
 * MFMA (the softmax / matrix-core balance).  They are not part of the
 * attention API.
 *
 * All pointers are device pointers; every call only enqueues on `stream`
 * (a hipStream_t, NULL = default) and returns 0, or a negative value for a
 * bad argument or launch failure.
 */
#ifndef HIFA4_PROBES_H_
#define HIFA4_PROBES_H_

#include <stdint.h>

#if defined(__GNUC__)
#define HIFA4_PROBE_API __attribute__((visibility("default")))
#else
#define HIFA4_PROBE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* One v_mfma_scale_f32_32x32x64_f8f6f4 (both operands FP4 E2M1) per wave.
 * a, b: [n_waves][64 lanes][4] dwords (the A / B operand registers of each
 * lane); sa, sb: [n_waves][64] scale registers; d: [n_waves][64][16] fp32
 * accumulator registers (C = 0).  opsel (0..3) is passed for both scales. */
HIFA4_PROBE_API int probe_mfma_fp4_32x32x64(const uint32_t* a, const uint32_t* b, const uint32_t* sa,
                            const uint32_t* sb, float* d, int n_waves, int opsel, void* stream);

/* Same for v_mfma_scale_f32_16x16x128_f8f6f4; d: [n_waves][64][4]. */
HIFA4_PROBE_API int probe_mfma_fp4_16x16x128(const uint32_t* a, const uint32_t* b, const uint32_t* sa,
                             const uint32_t* sb, float* d, int n_waves, int opsel, void* stream);

/* One v_mfma_f32_32x32x16_bf16 per wave: a, b [n_waves][64][8] bf16, d [n_waves][64][16]. */
HIFA4_PROBE_API int probe_mfma_bf16_32x32x16(const uint16_t* a, const uint16_t* b, float* d, int n_waves,
                             void* stream);

/* out[i] = v_cvt_scalef32_pk_fp4_f32(0, x[2i], x[2i+1], scale[i]) writing byte `sel`. */
HIFA4_PROBE_API int probe_cvt_pk_fp4(const float* x, const float* scale, uint32_t* out, int n, int sel,
                     void* stream);

/* v_permlane32_swap_b32 with both operands = x: out[2i], out[2i+1] are the two
 * results for element i = wave*64 + lane (x: [n_waves*64], out: [n_waves*64*2]). */
HIFA4_PROBE_API int probe_half_swap(const float* x, float* out, int n_waves, void* stream);

/* Throughput loops (n_blocks x 256 threads): 8 independent v_exp_f32 chains per
 * thread, or 4 independent FP4 32x32x64 MFMA chains per wave, iters times.
 * out: [n_blocks * 256] floats (keeps the work alive). */
HIFA4_PROBE_API int probe_exp2_rate(float* out, int n_blocks, int iters, void* stream);
HIFA4_PROBE_API int probe_mfma_rate(float* out, int n_blocks, int iters, void* stream);
/* Throughput of the 16 x 16 x 128 FP4 MFMA: 256-thread blocks, each wave runs eight
 * independent chains of `iters` MFMAs (65536 flops each); out[n_blocks * 256]. */
HIFA4_PROBE_API int probe_mfma16_rate(float* out, int n_blocks, int iters, void* stream);

/* Co-execution of FP4 MFMAs and vector work: n_blocks x 512 threads (two waves
 * per SIMD), per iteration 16 FP4 32x32x64 MFMAs (4 independent chains) and 32
 * exp2(fma) pairs (8 independent chains), iters times.  mode 0: MFMAs only;
 * 1: vector work only; 2: both in every wave, interleaved; 3: waves 0-3 the
 * MFMAs and waves 4-7 the vector work (one wave of each kind per SIMD).
 * out: [n_blocks * 512] floats (keeps the work alive).  Returns -1 on a bad
 * argument. */
HIFA4_PROBE_API int probe_coexec(float* out, int mode, int n_blocks, int iters, void* stream);

/* Issue cost of the softmax step's vector instructions: n_blocks x 512 threads
 * (two waves per SIMD), each wave runs iters iterations of 32 instructions on 8
 * independent chains.  mode 0: fma; 1: v_exp_f32; 2: exp and fma alternating;
 * 3: the 2-value FP4 convert (v_cvt_scalef32_pk_fp4_f32) and fma alternating;
 * 4: v_maximum3_f32; 5: convert and exp alternating; 6: waves 0-3 exp only,
 * waves 4-7 fma only (one wave of each kind per SIMD).  out: [n_blocks * 512]
 * floats (keeps the work alive).  Returns -1 on a bad argument. */
HIFA4_PROBE_API int probe_valu_rate(float* out, int mode, int n_blocks, int iters, void* stream);

/* The LDS transpose read of 16-bit elements (ds_read_b64_tr_b16): LDS holds
 * element i = i over 4096 16-bit elements; lane l (one wave) reads at element
 * offset addr[l] (device, 64 ints, each a multiple of 4 and at most 4092) and
 * writes its 4 results to out[4l .. 4l+3] (device, 256 shorts). */
HIFA4_PROBE_API int probe_lds_read_tr16(const int* addr, short* out, void* stream);

/* One wave of memory -> LDS buffer loads of `size` bytes per lane (1, 2, 4 or
 * 16), lane i reading src bytes [size*i, size*(i+1)) (src: 1024 bytes), with
 * M0 = LDS window + 64.  out: the 1088-byte window afterwards (pre-filled
 * with 0xEE), so the caller sees each lane's placement. */
HIFA4_PROBE_API int probe_lds_dma(const uint8_t* src, uint8_t* out, int size, void* stream);

/* Raw buffer range check with an SGPR offset: lane i loads the dword at
 * voffset 4i, soffset `soffset`, from a descriptor over src with
 * `num_records` bytes (src must hold soffset + 256 readable bytes).
 * out[0..64): register loads, out[64..128): the memory -> LDS form. */
HIFA4_PROBE_API int probe_buffer_range(const uint32_t* src, uint32_t* out, int soffset,
                                       int num_records, void* stream);

/* Streaming read: n_blocks x 256 threads read `bytes` (a multiple of 16) of
 * src in 16-byte words, grid-stride, four words in flight per thread, and
 * write the xor of every word each thread read to out[n_blocks * 256]
 * (which keeps the loads alive).  Timed over a buffer larger than the
 * last-level cache, it gives the HBM read rate a plain kernel reaches. */
HIFA4_PROBE_API int probe_stream_read(const void* src, size_t bytes, uint32_t* out, int n_blocks,
                                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HIFA4_PROBES_H_ */
