// quantize.hip -- Smooth-QK + MXFP4 quantisation of Q, K and V (gfx950).
//
// Method: "HiFA4: Training-Free 4-bit FlashAttention on Ascend HIF4 NPUs for
// LLM Inference", Abstract (Smooth-QK): queries are multiplied and keys
// divided by a static per-channel vector s after RoPE, which leaves Q K^T
// unchanged in exact arithmetic and moves quantisation difficulty from K to Q.
// Format: OCP MXFP4 (E2M1 elements, E8M0 scale per 32), the stand-in for the
// undefined HIF4 layout.
//
// One launch covers all three tensors; its grid is split in uniform ranges of
// workgroups (V token blocks, K rows, Q rows).  The work is HBM bound (2 bytes
// in, 17/32 byte out per element), so every access is coalesced across the
// wave:
//   - Q / K: four lanes share a 32-element block, each loading 16 contiguous
//     bytes (a wave reads 1 KB contiguous per instruction, four such loads in
//     flight per lane); the block max is two lane shuffles; each lane writes
//     its 4 code bytes, so a block's 16 code bytes and a wave's 256 bytes are
//     contiguous;
//   - V: one lane per (channel pair, 32-token block) reads the pair down the
//     32 tokens (a wave reads 256 contiguous bytes per token) and writes the
//     two channels' 16-byte code runs next to each other.
// The element encode is the gfx950 packed FP4 convert, which divides by the
// power-of-two block scale and rounds to nearest-even with saturation (the
// probes check it bit-for-bit against the CPU reference's encoder).
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


// Value of the lane selected by a DPP quad_perm control within each quad.
#define quad_xor(x, ctrl)                                                               \
  __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), (ctrl), 0xF, 0xF, false))


// Row blocks (blocks of 32 along the head dim): four lanes share a block,
// lane `lane4` handling elements 8*lane4 .. 8*lane4+7.  A lane processes
// kRowParts blocks, kThreads*4 parts apart, with every load issued before any
// use so that a wave keeps kRowParts KB of HBM reads in flight.
constexpr int kRowParts = 4;

struct RowPart {
  uint32_t orow;  // output row (b, h, t) with the token capacity applied
  uint32_t j0;    // first element of this lane's 8
  bool ok;
};

// Index arithmetic is 32-bit (the launcher checks the sizes fit), with the
// head dim a compile-time constant, so the per-part decode is a handful of
// integer ops rather than 64-bit divisions.
template <bool kBf16, int D>
__device__ __forceinline__ void quantise_rows(const uint16_t* __restrict__ x,
                                              const float* __restrict__ s, bool divide,
                                              uint32_t part0, uint32_t n_parts, uint32_t H,
                                              uint32_t S, uint32_t group, uint32_t cap,
                                              uint8_t* __restrict__ codes,
                                              uint8_t* __restrict__ scales) {
  constexpr uint32_t NB = D / 32;
  uint4 w[kRowParts];
  float4 f0[kRowParts], f1[kRowParts];
  RowPart rp[kRowParts];
#pragma unroll
  for (int r = 0; r < kRowParts; r++) {
    const uint32_t part = part0 + (uint32_t)r * kThreads;
    rp[r].ok = part < n_parts;
    const uint32_t blk = rp[r].ok ? part >> 2 : 0u;
    const uint32_t row = blk / NB;  // flattened (b, h, t)
    rp[r].j0 = (blk % NB) * 32u + 8u * (part & 3u);
    const uint32_t bh = row / S;
    const uint32_t t = row - bh * S;
    rp[r].orow = bh * cap + t;
    w[r] = rp[r].ok ? *reinterpret_cast<const uint4*>(x + (size_t)row * D + rp[r].j0)
                    : make_uint4(0, 0, 0, 0);
    if (s != nullptr) {
      const uint32_t hs = (bh % H) / group;
      const float4* sp = reinterpret_cast<const float4*>(s + hs * D + rp[r].j0);
      f0[r] = sp[0];
      f1[r] = sp[1];
    }
  }
#pragma unroll
  for (int r = 0; r < kRowParts; r++) {
    const uint32_t ws[4] = {w[r].x, w[r].y, w[r].z, w[r].w};
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = elem<kBf16>(ws[i] & 0xFFFFu);
      v[2 * i + 1] = elem<kBf16>(ws[i] >> 16);
    }
    if (s != nullptr) {
      const float ff[8] = {f0[r].x, f0[r].y, f0[r].z, f0[r].w, f1[r].x, f1[r].y, f1[r].z, f1[r].w};
#pragma unroll
      for (int i = 0; i < 8; i++) v[i] = divide ? v[i] / ff[i] : v[i] * ff[i];
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(v[i]));
    // the four lanes of a block are one DPP quad (consecutive, all valid or
    // all invalid): two quad permutes give the block max in every lane
    amax = fmaxf(amax, quad_xor(amax, 0xB1));  // lanes 1,0,3,2
    amax = fmaxf(amax, quad_xor(amax, 0x4E));  // lanes 2,3,0,1
    if (!rp[r].ok) continue;
    const uint32_t sb = e8m0_from_amax(amax);
    *reinterpret_cast<uint32_t*>(codes + (size_t)rp[r].orow * (D / 2) + rp[r].j0 / 2) =
        encode8(v, e8m0_to_float(sb));
    if ((rp[r].j0 & 31u) == 0) scales[(size_t)rp[r].orow * NB + rp[r].j0 / 32] = (uint8_t)sb;
  }
}

// One lane = channels (2c, 2c+1) of one 32-token block of one (b, h); tokens
// past S are zero.  Work item index: ((bh * nblk_valid) + blk) * (D/2) + c.
template <bool kBf16, int D>
__device__ __forceinline__ void quantise_v_pair(const uint16_t* __restrict__ x, uint32_t item,
                                                uint32_t S, uint32_t cap,
                                                uint8_t* __restrict__ codes,
                                                uint8_t* __restrict__ scales) {
  constexpr uint32_t HALF = D / 2;
  const uint32_t nblk_valid = (S + 31) / 32;
  const uint32_t c = item % HALF;
  const uint32_t rest = item / HALF;
  const uint32_t bh = rest / nblk_valid;
  const uint32_t blk = rest - bh * nblk_valid;
  const uint32_t t0 = blk * 32;
  const uint16_t* src = x + ((size_t)bh * S + t0) * D + 2 * c;
  float a[32], b[32];
#pragma unroll
  for (int k = 0; k < 32; k++) {
    uint32_t w = 0;
    if (t0 + k < S) w = *reinterpret_cast<const uint32_t*>(src + (size_t)k * D);
    a[k] = elem<kBf16>(w & 0xFFFFu);
    b[k] = elem<kBf16>(w >> 16);
  }
  float ma = 0.0f, mb = 0.0f;
#pragma unroll
  for (int k = 0; k < 32; k++) {
    ma = fmaxf(ma, fabsf(a[k]));
    mb = fmaxf(mb, fabsf(b[k]));
  }
  const uint32_t sa = e8m0_from_amax(ma), sbb = e8m0_from_amax(mb);
  const float fa = e8m0_to_float(sa), fb = e8m0_to_float(sbb);
  uint32_t ca[4], cb[4];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const float va[8] = {a[8 * q], a[8 * q + 1], a[8 * q + 2], a[8 * q + 3],
                         a[8 * q + 4], a[8 * q + 5], a[8 * q + 6], a[8 * q + 7]};
    const float vb[8] = {b[8 * q], b[8 * q + 1], b[8 * q + 2], b[8 * q + 3],
                         b[8 * q + 4], b[8 * q + 5], b[8 * q + 6], b[8 * q + 7]};
    ca[q] = encode8(va, fa);
    cb[q] = encode8(vb, fb);
  }
  const uint32_t nblk_cap = (cap + 31) / 32;
  const size_t ob = (size_t)bh * nblk_cap + blk;
  uint4* dst = reinterpret_cast<uint4*>(codes + (ob * D + 2 * c) * 16);
  dst[0] = make_uint4(ca[0], ca[1], ca[2], ca[3]);
  dst[1] = make_uint4(cb[0], cb[1], cb[2], cb[3]);
  *reinterpret_cast<uint16_t*>(scales + ob * D + 2 * c) = (uint16_t)(sa | (sbb << 8));
}

template <bool kBf16, int D>
__global__ __launch_bounds__(kThreads) void quantize_qkv_kernel(QuantizeArgs a) {
  // Grid order: V token blocks (the longest work items) first, then K, then
  // Q, so that the long items do not form the tail of the launch.
  const uint32_t wg = blockIdx.x;
  const uint32_t wg_v = (uint32_t)((a.items_v + kThreads - 1) / kThreads);
  const uint32_t wg_k = (uint32_t)a.wg_k;
  if (wg < wg_v) {
    const uint32_t item = wg * kThreads + threadIdx.x;
    if (item < (uint32_t)a.items_v)
      quantise_v_pair<kBf16, D>(a.v, item, a.Sk, a.cap, a.v_codes, a.v_scales);
  } else if (wg < wg_v + wg_k) {
    const uint32_t part0 = (wg - wg_v) * kThreads * kRowParts + threadIdx.x;
    quantise_rows<kBf16, D>(a.k, a.smooth, true, part0, (uint32_t)(4 * a.blocks_k), a.Hkv, a.Sk,
                            1, a.cap, a.k_codes, a.k_scales);
  } else {
    const uint32_t part0 = (wg - wg_v - wg_k) * kThreads * kRowParts + threadIdx.x;  // 4 parts per block
    quantise_rows<kBf16, D>(a.q, a.smooth, false, part0, (uint32_t)(4 * a.blocks_q), a.Hq, a.Sq,
                            a.Hq / a.Hkv, a.Sq, a.q_codes, a.q_scales);
  }
}

template <bool kBf16>
void launch_d(const QuantizeArgs& a, unsigned grid, hipStream_t stream) {
  switch (a.d) {
    case 64: hipLaunchKernelGGL((quantize_qkv_kernel<kBf16, 64>), dim3(grid), dim3(kThreads), 0, stream, a); break;
    case 128: hipLaunchKernelGGL((quantize_qkv_kernel<kBf16, 128>), dim3(grid), dim3(kThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL((quantize_qkv_kernel<kBf16, 256>), dim3(grid), dim3(kThreads), 0, stream, a); break;
  }
}

}  // namespace

hipError_t launch_quantize_qkv(QuantizeArgs a, bool bf16, hipStream_t stream) {
  const int64_t per_wg = (int64_t)kThreads * kRowParts;
  a.wg_q = a.q ? (4 * a.blocks_q + per_wg - 1) / per_wg : 0;
  a.wg_k = a.k ? (4 * a.blocks_k + per_wg - 1) / per_wg : 0;
  a.items_v = a.v ? (int64_t)a.B * a.Hkv * ((a.Sk + 31) / 32) * (a.d / 2) : 0;
  const int64_t wg_v = (a.items_v + kThreads - 1) / kThreads;
  const int64_t total = a.wg_q + a.wg_k + wg_v;
  if (total == 0) return hipSuccess;
  // 32-bit index arithmetic inside the kernel
  const int64_t lim = 0x7FFFFFFF;
  if (total > lim / (kThreads * kRowParts) || 4 * a.blocks_q > lim || 4 * a.blocks_k > lim ||
      a.items_v > lim || (int64_t)a.B * a.Hkv * a.cap > lim || (int64_t)a.B * a.Hq * a.Sq > lim)
    return hipErrorInvalidConfiguration;
  if (bf16)
    launch_d<true>(a, (unsigned)total, stream);
  else
    launch_d<false>(a, (unsigned)total, stream);
  return hipGetLastError();
}

}  // namespace hifa4
