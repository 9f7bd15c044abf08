// quantize.hip -- Smooth-QK + MXFP4 quantisation of Q, K and V (gfx950).
//
// Method: "HiFA4: Training-Free 4-bit FlashAttention on Ascend HIF4 NPUs for
// LLM Inference", Abstract (Smooth-QK): queries are multiplied and keys
// divided by a static per-channel vector s after RoPE, which leaves Q K^T
// unchanged in exact arithmetic and moves quantisation difficulty from K to Q.
// Format: OCP MXFP4 (E2M1 elements, E8M0 scale per 32), the stand-in for the
// undefined HIF4 layout.
//
// One launch covers all three tensors; its grid is split in three uniform
// ranges of workgroups (Q rows, K rows, V token blocks).  The work is HBM
// bound: 2 bytes in and 17/32 byte out per element, so every store is a
// contiguous 16-byte code chunk or a run of scale bytes across the wave.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "launch.hpp"

// Bit-exact parity with a reference quantiser needs IEEE multiply and divide
// with no contraction.
#pragma clang fp contract(off)

namespace hifa4 {
namespace {

constexpr int kThreads = 256;

template <bool kBf16>
__device__ __forceinline__ float elem(uint32_t bits16) {
  if constexpr (kBf16) {
    return bf16_bits_to_float(bits16);
  } else {
    return __half2float(__ushort_as_half((unsigned short)bits16));
  }
}

// E2M1 code of x / 2^e given neg_e = -e: the magnitude is compared with the
// seven decision points between neighbouring E2M1 values; at an exact
// midpoint the comparison direction picks the even code (0.25 -> 0,
// 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2.0, 2.5 -> 2.0, 3.5 -> 4.0, 5 -> 4.0);
// above 5 everything clamps to 6.0.  The sign bit of x is kept (-0 -> 0x8).
__device__ __forceinline__ uint32_t e2m1_code(float x, int neg_e) {
  float y = ldexpf(fabsf(x), neg_e);
  uint32_t c = (uint32_t)(y > 0.25f) + (uint32_t)(y >= 0.75f) + (uint32_t)(y > 1.25f) +
               (uint32_t)(y >= 1.75f) + (uint32_t)(y > 2.5f) + (uint32_t)(y >= 3.5f) +
               (uint32_t)(y > 5.0f);
  return c | ((__float_as_uint(x) >> 28) & 8u);
}

// Quantise 32 fp32 values: 16 code bytes + the E8M0 byte.
__device__ __forceinline__ uint4 quantise32(const float (&v)[32], uint32_t& scale_byte) {
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; j++) amax = fmaxf(amax, fabsf(v[j]));
  scale_byte = e8m0_from_amax(amax);
  const int neg_e = 127 - (int)scale_byte;
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) acc |= e2m1_code(v[8 * q + i], neg_e) << (4 * i);
    w[q] = acc;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// One thread = one 32-element block of one row (blocks along the head dim).
template <bool kBf16>
__device__ void quantise_row_block(const uint16_t* __restrict__ x, const float* __restrict__ s,
                                   bool divide, int64_t blk, int H, int S, int d, int group,
                                   int cap, uint8_t* __restrict__ codes,
                                   uint8_t* __restrict__ scales) {
  const int nb = d / 32;
  const int64_t row = blk / nb;  // flattened (b, h, t)
  const int j0 = (int)(blk % nb) * 32;
  const int t = (int)(row % S);
  const int64_t bh = row / S;
  const int h = (int)(bh % H);
  const uint4* src = reinterpret_cast<const uint4*>(x + row * d + j0);
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    uint4 w = src[q];
    uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[8 * q + 2 * i] = elem<kBf16>(ws[i] & 0xFFFFu);
      v[8 * q + 2 * i + 1] = elem<kBf16>(ws[i] >> 16);
    }
  }
  if (s != nullptr) {
    const float4* sp = reinterpret_cast<const float4*>(s + (int64_t)(h / group) * d + j0);
#pragma unroll
    for (int q = 0; q < 8; q++) {
      float4 f = sp[q];
      float ff[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
      for (int i = 0; i < 4; i++) v[4 * q + i] = divide ? v[4 * q + i] / ff[i] : v[4 * q + i] * ff[i];
    }
  }
  uint32_t sb;
  uint4 c = quantise32(v, sb);
  const int64_t orow = bh * cap + t;
  *reinterpret_cast<uint4*>(codes + orow * (d / 2) + j0 / 2) = c;
  scales[orow * nb + j0 / 32] = (uint8_t)sb;
}

// One workgroup = kThreads / d consecutive 32-token blocks of one (b, h);
// thread = one channel of one block.  The token tile is staged through LDS
// with coalesced 16-byte loads; each thread then reads its channel's column
// (a contiguous row of the wave per step, so no bank conflicts).
template <bool kBf16>
__device__ void quantise_v_tile(const uint16_t* __restrict__ x, int64_t wg, int S, int d, int cap,
                                uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                uint16_t* lds) {
  const int blocks_per_wg = kThreads / d;
  const int nblk_valid = (S + 31) / 32;
  const int wg_per_head = (nblk_valid + blocks_per_wg - 1) / blocks_per_wg;
  const int64_t bh = wg / wg_per_head;
  const int blk0 = (int)(wg % wg_per_head) * blocks_per_wg;
  const int t0 = blk0 * 32;
  const int ntok = blocks_per_wg * 32;  // tokens staged
  const uint16_t* xh = x + bh * (int64_t)S * d;
  // stage ntok x d elements (8192 for every d) as 16-byte chunks
  const int chunks = ntok * d / 8;
  for (int i = threadIdx.x; i < chunks; i += kThreads) {
    const int tok = (i * 8) / d;
    const int c8 = (i * 8) % d;
    uint4 w = make_uint4(0, 0, 0, 0);
    if (t0 + tok < S) w = *reinterpret_cast<const uint4*>(xh + (int64_t)(t0 + tok) * d + c8);
    *reinterpret_cast<uint4*>(lds + tok * d + c8) = w;
  }
  __syncthreads();
  const int lb = threadIdx.x / d;  // local block
  const int ch = threadIdx.x % d;
  const int blk = blk0 + lb;
  if (blk >= nblk_valid) return;
  float v[32];
#pragma unroll
  for (int k = 0; k < 32; k++) v[k] = elem<kBf16>(lds[(lb * 32 + k) * d + ch]);
  uint32_t sb;
  uint4 c = quantise32(v, sb);
  const int nblk_cap = (cap + 31) / 32;
  const int64_t ob = bh * nblk_cap + blk;
  *reinterpret_cast<uint4*>(codes + (ob * d + ch) * 16) = c;
  scales[ob * d + ch] = (uint8_t)sb;
}

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void quantize_qkv_kernel(QuantizeArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[8192];
  const int64_t wg = blockIdx.x;
  if (wg < a.wg_q) {
    const int64_t blk = wg * kThreads + threadIdx.x;
    if (blk < a.blocks_q)
      quantise_row_block<kBf16>(a.q, a.smooth, false, blk, a.Hq, a.Sq, a.d, a.Hq / a.Hkv, a.Sq,
                                a.q_codes, a.q_scales);
  } else if (wg < a.wg_q + a.wg_k) {
    const int64_t blk = (wg - a.wg_q) * kThreads + threadIdx.x;
    if (blk < a.blocks_k)
      quantise_row_block<kBf16>(a.k, a.smooth, true, blk, a.Hkv, a.Sk, a.d, 1, a.cap, a.k_codes,
                                a.k_scales);
  } else {
    quantise_v_tile<kBf16>(a.v, wg - a.wg_q - a.wg_k, a.Sk, a.d, a.cap, a.v_codes, a.v_scales,
                           lds);
  }
}

}  // namespace

hipError_t launch_quantize_qkv(QuantizeArgs a, bool bf16, hipStream_t stream) {
  a.wg_q = a.q ? (a.blocks_q + kThreads - 1) / kThreads : 0;
  a.wg_k = a.k ? (a.blocks_k + kThreads - 1) / kThreads : 0;
  int64_t wg_v = 0;
  if (a.v) {
    const int blocks_per_wg = kThreads / a.d;
    const int nblk_valid = (a.Sk + 31) / 32;
    wg_v = (int64_t)a.B * a.Hkv * ((nblk_valid + blocks_per_wg - 1) / blocks_per_wg);
  }
  const int64_t total = a.wg_q + a.wg_k + wg_v;
  if (total == 0) return hipSuccess;
  if (total > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (bf16)
    hipLaunchKernelGGL(quantize_qkv_kernel<true>, dim3((unsigned)total), dim3(kThreads), 0, stream,
                       a);
  else
    hipLaunchKernelGGL(quantize_qkv_kernel<false>, dim3((unsigned)total), dim3(kThreads), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace hifa4
