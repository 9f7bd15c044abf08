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
// lane `lane4` handling elements 8*lane4 .. 8*lane4+7.  A lane may process
// kRowParts blocks, kThreads parts apart (the same 8 channels of rows that
// far apart), with every load issued before any use.  Without smoothing one
// part per lane was fastest (K, V of the Qwen3-8B layer: 6.7 us with 1 part,
// 7.0 with 2, 7.5 with 4, 9.0 with 8: more, shorter workgroups finish a single
// round sooner).  Since K / s goes through a per-workgroup table of double
// reciprocals, two parts halve the table builds per element: K, V of the
// Gemma2-9B-shaped layer between attention launches 43.7 -> 37.8 us (4 parts:
// 38.0), the Qwen3- and Llama-shaped layers unchanged within noise.
constexpr int kRowParts = 2;

struct RowPart {
  uint32_t orow;  // output row (b, h, t) with the token capacity applied
  uint32_t j0;    // first element of this lane's 8
  uint32_t t;     // token of the row
  bool ok;
};

// Rotate-half RoPE of the lane's 8 elements j0 .. j0+7: the partner elements
// (j +- d/2) belong to the lane 2*NB parts away in the same row (a row's
// 4*NB parts are consecutive lanes of one wave), exchanged as raw words.  The
// table entries are loaded first (rope_load, issued with the row loads).
struct RopeCS {
  float4 c0, c1, s0, s1;
};

template <int D>
__device__ __forceinline__ RopeCS rope_load(uint32_t j0, uint32_t pos,
                                            const float* __restrict__ cosv,
                                            const float* __restrict__ sinv) {
  constexpr uint32_t HALF = D / 2;
  const uint32_t jj = j0 % HALF;
  const float4* cp = reinterpret_cast<const float4*>(cosv + (size_t)pos * HALF + jj);
  const float4* sp = reinterpret_cast<const float4*>(sinv + (size_t)pos * HALF + jj);
  return RopeCS{cp[0], cp[1], sp[0], sp[1]};
}

template <bool kBf16, int D>
__device__ __forceinline__ void rope8(float (&v)[8], const uint4& w, uint32_t j0,
                                      const RopeCS& cs) {
  constexpr int NB = D / 32;
  constexpr uint32_t HALF = D / 2;
  const uint32_t pw[4] = {(uint32_t)__shfl_xor((int)w.x, 2 * NB), (uint32_t)__shfl_xor((int)w.y, 2 * NB),
                          (uint32_t)__shfl_xor((int)w.z, 2 * NB), (uint32_t)__shfl_xor((int)w.w, 2 * NB)};
  float u[8];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    u[2 * i] = elem<kBf16>(pw[i] & 0xFFFFu);
    u[2 * i + 1] = elem<kBf16>(pw[i] >> 16);
  }
  const float4 c0 = cs.c0, c1 = cs.c1, s0 = cs.s0, s1 = cs.s1;
  const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  const bool first = j0 < HALF;  // own element is x[j] (partner x[j + d/2]) or the reverse
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float own = v[i] * c[i];
    const float other = u[i] * sn[i];
    v[i] = first ? own - other : own + other;
  }
}

// Index arithmetic is 32-bit (the launcher checks the sizes fit), with the
// head dim a compile-time constant, so the per-part decode is a handful of
// integer ops rather than 64-bit divisions.
// Cache append (kAppend): token t of sequence b sits at L_b + t, with L_b the
// sequence's current length from `lens` (clamped to [0, kv_cap]); with
// offset_rows the output is cache row L_b + t and rows past the capacity are
// not written, else row t.  Table rows are clamped to max_pos, so a length
// past the tables reads no memory outside them.
struct AppendRows {
  const int32_t* lens;
  uint32_t kv_cap;
  bool offset_rows;
  uint32_t max_pos;
};

// kRcp: the division by s uses the workgroup's table of reciprocals (rcp,
// the rows of heads bh0 and bh0 + 1), see quantize_qkv_kernel; `fill` builds
// it, called between the loads and their first use.
struct NoFill {
  __device__ void operator()() const {}
};
template <bool kBf16, int D, bool kRope, bool kAppend = false, bool kRcp = false,
          typename Fill = NoFill>
__device__ __forceinline__ void quantise_rows(const uint16_t* __restrict__ x,
                                              const float* __restrict__ s, bool divide,
                                              uint32_t bias, uint32_t part0, uint32_t n_parts, uint32_t H,
                                              uint32_t S, uint32_t group, uint32_t cap,
                                              uint8_t* __restrict__ codes,
                                              uint8_t* __restrict__ scales,
                                              const float* __restrict__ rope_cos,
                                              const float* __restrict__ rope_sin,
                                              uint32_t pos0, AppendRows ap = {},
                                              const double* rcp = nullptr, uint32_t bh0 = 0,
                                              Fill fill = {}) {
  constexpr uint32_t NB = D / 32;
  uint4 w[kRowParts];
  float4 f0[kRowParts], f1[kRowParts];
  uint32_t rrow[kRowParts];  // kRcp: the lane's row of reciprocals
  RowPart rp[kRowParts];
  RopeCS cs[kRowParts];
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
    rp[r].t = t;
    w[r] = rp[r].ok ? *reinterpret_cast<const uint4*>(x + (size_t)row * D + rp[r].j0)
                    : make_uint4(0, 0, 0, 0);
    if constexpr (kAppend) {
      const int32_t l = ap.lens[bh / H];
      const uint32_t L = l < 0 ? 0u : min((uint32_t)l, ap.kv_cap);
      rp[r].t = L + t;
      if (ap.offset_rows) {
        rp[r].orow += L;
        // a row is written only inside the cache (uniform over the row's lanes)
        rp[r].ok = rp[r].ok && L + t < ap.kv_cap;
      }
    }
    if constexpr (kRope) {
      const uint32_t pos = kAppend ? min(pos0 + rp[r].t, ap.max_pos) : pos0 + rp[r].t;
      cs[r] = rope_load<D>(rp[r].j0, pos, rope_cos, rope_sin);
    }
    if constexpr (kRcp) {
      rrow[r] = rp[r].ok ? (bh - bh0) * D : 0u;
    } else if (s != nullptr) {
      const uint32_t hs = (bh % H) / group;
      const float4* sp = reinterpret_cast<const float4*>(s + hs * D + rp[r].j0);
      f0[r] = sp[0];
      f1[r] = sp[1];
    }
  }
  if constexpr (kRcp) fill();  // the table, while the row loads are in flight
#pragma unroll
  for (int r = 0; r < kRowParts; r++) {
    const uint32_t ws[4] = {w[r].x, w[r].y, w[r].z, w[r].w};
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = elem<kBf16>(ws[i] & 0xFFFFu);
      v[2 * i + 1] = elem<kBf16>(ws[i] >> 16);
    }
    // RoPE first (every lane takes part in the partner exchange), then Smooth-QK
    if constexpr (kRope) rope8<kBf16, D>(v, w[r], rp[r].j0, cs[r]);
    if constexpr (kRcp) {
      // x / s as RN32(x * RN64(1 / s)), the same bits as the fp32 division
      // (see quantize_qkv_kernel)
      const double* rr = rcp + rrow[r] + rp[r].j0;
#pragma unroll
      for (int i = 0; i < 8; i++) v[i] = (float)((double)v[i] * rr[i]);
    } else if (s != nullptr) {
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
    const uint32_t sb = e8m0_from_amax(amax, bias);
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
                                                uint8_t* __restrict__ scales, uint32_t bias) {
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
  const uint32_t sa = e8m0_from_amax(ma, bias), sbb = e8m0_from_amax(mb, bias);
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

template <bool kBf16, int D, bool kRope>
__global__ __launch_bounds__(kThreads) void quantize_qkv_kernel(QuantizeArgs a) {
  // Grid order: V token blocks (the longest work items) first, then K, then
  // Q, so that the long items do not form the tail of the launch.
  const uint32_t wg = blockIdx.x;
  const uint32_t wg_v = (uint32_t)((a.items_v + kThreads - 1) / kThreads);
  const uint32_t wg_k = (uint32_t)a.wg_k;
  if (wg < wg_v) {
    const uint32_t item = wg * kThreads + threadIdx.x;
    if (item < (uint32_t)a.items_v)
      quantise_v_pair<kBf16, D>(a.v, item, a.Sk, a.cap, a.v_codes, a.v_scales, a.v_bias);
  } else if (wg < wg_v + wg_k) {
    const uint32_t part0 = (wg - wg_v) * kThreads * kRowParts + threadIdx.x;
    const uint32_t n_parts = (uint32_t)(4 * a.blocks_k);
    // K / s.  Each element's fp32 quotient is computed as RN32(x * RN64(1/s)):
    // the double product is within 2^-52 (relative) of x / s, while x / s
    // (two binary32 operands) is never a binary32 rounding midpoint and, when
    // it is not one, lies at least 2^-49 (relative) from one, so the final
    // rounding is that of the fp32 division, bit for bit.  The reciprocals
    // depend only on the channel: the workgroup computes them once, for the
    // (at most two) heads its rows belong to, instead of one fp32 division per
    // element; the table is built while the row loads are in flight (K and V
    // of the Gemma2-9B-shaped layer, inputs not in the last-level cache:
    // 40.1 -> 38.8 us).
    constexpr uint32_t NB = D / 32;
    const uint32_t p_first = (wg - wg_v) * kThreads * kRowParts;
    const uint32_t p_last = min(p_first + kThreads * kRowParts, n_parts) - 1;
    const uint32_t bh0 = (p_first >> 2) / NB / (uint32_t)a.Sk;
    const uint32_t bh1 = (p_last >> 2) / NB / (uint32_t)a.Sk;
    if (a.smooth != nullptr && bh1 <= bh0 + 1) {
      __shared__ double rcp[2 * D];
      auto fill = [&]() {
        for (uint32_t i = threadIdx.x; i < (bh1 - bh0 + 1) * D; i += kThreads) {
          const uint32_t hs = (bh0 + i / D) % (uint32_t)a.Hkv;
          rcp[i] = 1.0 / (double)a.smooth[hs * D + i % D];
        }
        __syncthreads();
      };
      quantise_rows<kBf16, D, kRope, false, true>(a.k, a.smooth, true, a.k_bias, part0, n_parts,
                                                  a.Hkv, a.Sk, 1, a.cap, a.k_codes, a.k_scales,
                                                  a.rope_cos, a.rope_sin, (uint32_t)a.k_pos0, {},
                                                  rcp, bh0, fill);
    } else {
      quantise_rows<kBf16, D, kRope>(a.k, a.smooth, true, a.k_bias, part0, n_parts, a.Hkv, a.Sk, 1,
                                     a.cap, a.k_codes, a.k_scales, a.rope_cos, a.rope_sin,
                                     (uint32_t)a.k_pos0);
    }
  } else {
    const uint32_t part0 = (wg - wg_v - wg_k) * kThreads * kRowParts + threadIdx.x;  // 4 parts per block
    quantise_rows<kBf16, D, kRope>(a.q, a.smooth, false, a.q_bias, part0, (uint32_t)(4 * a.blocks_q), a.Hq,
                                   a.Sq, a.Hq / a.Hkv, a.Sq, a.q_codes, a.q_scales, a.rope_cos,
                                   a.rope_sin, (uint32_t)a.q_pos0);
  }
}

template <bool kBf16, bool kRope>
void launch_d(const QuantizeArgs& a, unsigned grid, hipStream_t stream) {
  switch (a.d) {
    case 64: hipLaunchKernelGGL((quantize_qkv_kernel<kBf16, 64, kRope>), dim3(grid), dim3(kThreads), 0, stream, a); break;
    case 128: hipLaunchKernelGGL((quantize_qkv_kernel<kBf16, 128, kRope>), dim3(grid), dim3(kThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL((quantize_qkv_kernel<kBf16, 256, kRope>), dim3(grid), dim3(kThreads), 0, stream, a); break;
  }
}

// ---------------------------------------------------------------------------
// KV-cache append for decode.  New K rows are rotated, smoothed and quantised
// into cache rows L_b .. L_b + n - 1 (the row layout needs nothing else).  A
// value block holds 32 consecutive tokens of one channel under one scale, so
// a new token in a partly filled block changes that block's scale: the block
// is quantised again from the raw values of its earlier tokens, which the
// caller's tail buffer keeps ([B][Hkv][32][d], slot = token % 32).  One lane
// owns a (b, g, channel pair) for every block the append touches; it reads the
// old tail slots before it writes new ones, and no other lane touches them, so
// the buffer is updated in place.  The cache then equals a one-shot
// quantisation of the whole sequence.
template <bool kBf16, int D>
__device__ __forceinline__ void append_v_pair(const AppendArgs& a, uint32_t item) {
  constexpr uint32_t HALF = D / 2;
  const uint32_t c = item % HALF;
  const uint32_t bh = item / HALF;
  const uint32_t b = bh / (uint32_t)a.Hkv;
  const uint32_t cap = (uint32_t)a.cap;
  const int32_t l = a.lens[b];
  const uint32_t L = l < 0 ? 0u : min((uint32_t)l, cap);
  const uint32_t end = min(L + (uint32_t)a.n_new, cap);
  if (bh % (uint32_t)a.Hkv == 0 && c == 0 && a.lens_out) a.lens_out[b] = (int32_t)end;
  if (end <= L) return;
  const uint16_t* src = a.v + (size_t)bh * a.n_new * D + 2 * c;
  uint32_t* tail = reinterpret_cast<uint32_t*>(a.v_tail + (size_t)bh * 32 * D + 2 * c);
  const uint32_t nblk_cap = (cap + 31) / 32;
  for (uint32_t blk = L / 32; blk <= (end - 1) / 32; blk++) {
    const uint32_t t0 = blk * 32;
    uint32_t w[32];
#pragma unroll
    for (int k = 0; k < 32; k++) {
      const uint32_t tok = t0 + k;
      w[k] = 0;
      if (tok < L)
        w[k] = tail[(size_t)k * HALF];  // earlier token of this block
      else if (tok < end)
        w[k] = *reinterpret_cast<const uint32_t*>(src + (size_t)(tok - L) * D);
    }
    float va[32], vb[32];
    float ma = 0.0f, mb = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; k++) {
      va[k] = elem<kBf16>(w[k] & 0xFFFFu);
      vb[k] = elem<kBf16>(w[k] >> 16);
      ma = fmaxf(ma, fabsf(va[k]));
      mb = fmaxf(mb, fabsf(vb[k]));
    }
    const uint32_t sa = e8m0_from_amax(ma, a.v_bias), sbb = e8m0_from_amax(mb, a.v_bias);
    const float fa = e8m0_to_float(sa), fb = e8m0_to_float(sbb);
    uint32_t ca[4], cb[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const float xa[8] = {va[8 * q], va[8 * q + 1], va[8 * q + 2], va[8 * q + 3],
                           va[8 * q + 4], va[8 * q + 5], va[8 * q + 6], va[8 * q + 7]};
      const float xb[8] = {vb[8 * q], vb[8 * q + 1], vb[8 * q + 2], vb[8 * q + 3],
                           vb[8 * q + 4], vb[8 * q + 5], vb[8 * q + 6], vb[8 * q + 7]};
      ca[q] = encode8(xa, fa);
      cb[q] = encode8(xb, fb);
    }
    const size_t ob = (size_t)bh * nblk_cap + blk;
    uint4* dst = reinterpret_cast<uint4*>(a.v_codes + (ob * D + 2 * c) * 16);
    dst[0] = make_uint4(ca[0], ca[1], ca[2], ca[3]);
    dst[1] = make_uint4(cb[0], cb[1], cb[2], cb[3]);
    *reinterpret_cast<uint16_t*>(a.v_scales + ob * D + 2 * c) = (uint16_t)(sa | (sbb << 8));
    // the block still open after the append keeps its new tokens' raw values
    if (end % 32 != 0 && blk == end / 32) {
#pragma unroll
      for (int k = 0; k < 32; k++)
        if (t0 + k >= L && t0 + k < end) tail[(size_t)k * HALF] = w[k];
    }
  }
}

template <bool kBf16, int D, bool kRope>
__global__ __launch_bounds__(kThreads) void kv_append_kernel(AppendArgs a) {
  const uint32_t wg = blockIdx.x;
  const uint32_t wg_v = (uint32_t)((a.items_v + kThreads - 1) / kThreads);
  const uint32_t wg_k = (uint32_t)a.wg_k;
  const uint32_t max_pos = (uint32_t)(a.n_pos > 0 ? a.n_pos - 1 : 0);
  if (wg < wg_v) {
    const uint32_t item = wg * kThreads + threadIdx.x;
    if (item < (uint32_t)a.items_v) append_v_pair<kBf16, D>(a, item);
  } else if (wg < wg_v + wg_k) {
    const uint32_t part0 = (wg - wg_v) * kThreads * kRowParts + threadIdx.x;
    quantise_rows<kBf16, D, kRope, true>(
        a.k, a.smooth, true, a.k_bias, part0, (uint32_t)(4 * a.blocks_k), a.Hkv, a.n_new, 1, a.cap,
        a.k_codes, a.k_scales, a.rope_cos, a.rope_sin, (uint32_t)a.k_pos0,
        AppendRows{a.lens, (uint32_t)a.cap, true, max_pos});
  } else {
    const uint32_t part0 = (wg - wg_v - wg_k) * kThreads * kRowParts + threadIdx.x;
    quantise_rows<kBf16, D, kRope, true>(
        a.q, a.smooth, false, a.q_bias, part0, (uint32_t)(4 * a.blocks_q), a.Hq, a.n_new, a.Hq / a.Hkv,
        a.n_new, a.q_codes, a.q_scales, a.rope_cos, a.rope_sin, (uint32_t)a.q_pos0,
        AppendRows{a.lens, (uint32_t)a.cap, false, max_pos});
  }
}

template <bool kBf16, bool kRope>
void launch_append_d(const AppendArgs& a, unsigned grid, hipStream_t stream) {
  switch (a.d) {
    case 64: hipLaunchKernelGGL((kv_append_kernel<kBf16, 64, kRope>), dim3(grid), dim3(kThreads), 0, stream, a); break;
    case 128: hipLaunchKernelGGL((kv_append_kernel<kBf16, 128, kRope>), dim3(grid), dim3(kThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL((kv_append_kernel<kBf16, 256, kRope>), dim3(grid), dim3(kThreads), 0, stream, a); break;
  }
}

// ---------------------------------------------------------------------------
// Offline Smooth-QK calibration (Abstract, Smooth-QK: s is static, taken from
// calibration activations): per KV head g and channel j, the maxima of |K| and
// of |Q| over the heads of g's query group, every batch entry and token, then
// s = (max|K| / max|Q|)^alpha in fp64, rounded to fp32; s = 1 where either
// maximum is zero.  Optionally the same rotate-half RoPE as the quantiser is
// applied first, since s is defined on post-RoPE activations.
//
// Pass 1 (calib_max_kernel): one workgroup per (tensor, b, h, 256-token
// chunk) with the quantiser's row layout (d/8 lanes per row, 16 bytes each);
// per-lane maxima, an LDS reduction over the workgroup's rows, then one
// unsigned atomic max per channel into the workspace (|x| is non-negative, so
// its bit pattern orders like its value; NaN never enters since fmaxf drops
// it).  Pass 2 (calib_finish_kernel) forms s.  The workspace is cleared by a
// fill kernel first.
constexpr int kCalibTokens = 256;

__global__ __launch_bounds__(kThreads) void calib_clear_kernel(uint32_t* ws, int n) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) ws[i] = 0u;
}

template <bool kBf16, int D, bool kRope>
__global__ __launch_bounds__(kThreads) void calib_max_kernel(CalibrateArgs a, uint32_t* ws) {
  constexpr int LPR = D / 8;          // lanes per row
  constexpr int RPI = kThreads / LPR;  // rows per pass of the workgroup
  constexpr int U = 4;                 // passes with loads in flight
  __shared__ float red[RPI][D];
  const uint32_t nch = (uint32_t)(a.S + kCalibTokens - 1) / kCalibTokens;
  const uint32_t items_k = (uint32_t)a.B * a.Hkv * nch;
  uint32_t item = blockIdx.x;
  const bool is_q = item >= items_k;
  if (is_q) item -= items_k;
  const uint32_t H = is_q ? a.Hq : a.Hkv;
  const uint32_t bh = item / nch;
  const uint32_t t0 = (item - bh * nch) * kCalibTokens;
  const uint32_t g = is_q ? (bh % H) / (a.Hq / a.Hkv) : bh % H;
  const uint16_t* x = (is_q ? a.q : a.k) + (size_t)bh * a.S * D;
  const int pos0 = is_q ? a.q_pos0 : a.k_pos0;
  const uint32_t r0 = threadIdx.x / LPR;
  const uint32_t j0 = (threadIdx.x % LPR) * 8;
  const uint32_t t_end = min((uint32_t)a.S, t0 + kCalibTokens);
  float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (uint32_t tb = t0; tb < t_end; tb += RPI * U) {
    uint4 w[U];
    uint32_t tt[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      tt[u] = tb + u * RPI + r0;
      // every lane of a row shares its token, so a row is valid or not as a whole
      w[u] = tt[u] < t_end ? *reinterpret_cast<const uint4*>(x + (size_t)tt[u] * D + j0)
                           : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      const uint32_t ws4[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
      float v[8];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        v[2 * i] = elem<kBf16>(ws4[i] & 0xFFFFu);
        v[2 * i + 1] = elem<kBf16>(ws4[i] >> 16);
      }
      if constexpr (kRope)  // zeros rotate to zeros; invalid rows use position pos0
        rope8<kBf16, D>(v, w[u], j0,
                        rope_load<D>(j0, pos0 + (tt[u] < t_end ? tt[u] : 0u), a.rope_cos,
                                     a.rope_sin));
#pragma unroll
      for (int i = 0; i < 8; i++) m[i] = fmaxf(m[i], fabsf(v[i]));
    }
  }
#pragma unroll
  for (int i = 0; i < 8; i++) red[r0][j0 + i] = m[i];
  __syncthreads();
  if (threadIdx.x < D) {
    float mx = 0.0f;
#pragma unroll
    for (int r = 0; r < RPI; r++) mx = fmaxf(mx, red[r][threadIdx.x]);
    if (mx > 0.0f)
      atomicMax(ws + (is_q ? (size_t)a.Hkv * D : 0) + (size_t)g * D + threadIdx.x,
                __float_as_uint(mx));
  }
}

__global__ __launch_bounds__(kThreads) void calib_finish_kernel(const uint32_t* ws, float* s,
                                                                int n, double alpha) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  const double km = (double)__uint_as_float(ws[i]);
  const double qm = (double)__uint_as_float(ws[n + i]);
  s[i] = (qm > 0.0 && km > 0.0) ? (float)pow(km / qm, alpha) : 1.0f;
}

template <bool kBf16, bool kRope>
void launch_calib_d(const CalibrateArgs& a, unsigned grid, uint32_t* ws, hipStream_t stream) {
  switch (a.d) {
    case 64: hipLaunchKernelGGL((calib_max_kernel<kBf16, 64, kRope>), dim3(grid), dim3(kThreads), 0, stream, a, ws); break;
    case 128: hipLaunchKernelGGL((calib_max_kernel<kBf16, 128, kRope>), dim3(grid), dim3(kThreads), 0, stream, a, ws); break;
    default: hipLaunchKernelGGL((calib_max_kernel<kBf16, 256, kRope>), dim3(grid), dim3(kThreads), 0, stream, a, ws); break;
  }
}

}  // namespace

hipError_t launch_kv_append(AppendArgs a, bool bf16, hipStream_t stream) {
  const int64_t per_wg = (int64_t)kThreads * kRowParts;
  const int64_t NB = a.d / 32;
  a.blocks_k = (int64_t)a.B * a.Hkv * a.n_new * NB;
  a.blocks_q = a.q ? (int64_t)a.B * a.Hq * a.n_new * NB : 0;
  a.wg_k = (4 * a.blocks_k + per_wg - 1) / per_wg;
  a.wg_q = (4 * a.blocks_q + per_wg - 1) / per_wg;
  a.items_v = (int64_t)a.B * a.Hkv * (a.d / 2);
  const int64_t wg_v = (a.items_v + kThreads - 1) / kThreads;
  const int64_t total = wg_v + a.wg_k + a.wg_q;
  if (a.B == 0) return hipSuccess;
  // 32-bit index arithmetic inside the kernel
  const int64_t lim = 0x7FFFFFFF;
  if (total > lim / (kThreads * kRowParts) || 4 * a.blocks_q > lim || 4 * a.blocks_k > lim ||
      (int64_t)a.B * a.Hkv * a.cap > lim || (int64_t)a.cap + a.n_new > lim ||
      (int64_t)a.B * a.Hq * a.n_new > lim)
    return hipErrorInvalidConfiguration;
  const bool rope = a.rope_cos != nullptr;
  if (bf16 && !rope)
    launch_append_d<true, false>(a, (unsigned)total, stream);
  else if (!rope)
    launch_append_d<false, false>(a, (unsigned)total, stream);
  else if (bf16)
    launch_append_d<true, true>(a, (unsigned)total, stream);
  else
    launch_append_d<false, true>(a, (unsigned)total, stream);
  return hipGetLastError();
}

hipError_t launch_smooth_calibrate(const CalibrateArgs& a, bool bf16, hipStream_t stream) {
  const int n = a.Hkv * a.d;
  uint32_t* ws = a.workspace;
  const int64_t nch = (a.S + kCalibTokens - 1) / kCalibTokens;
  const int64_t items = (int64_t)a.B * (a.Hq + a.Hkv) * nch;
  // 32-bit item and token arithmetic inside the kernel
  if (items > 0x7FFFFFFF || (int64_t)a.S + kCalibTokens > 0x7FFFFFFF)
    return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(calib_clear_kernel, dim3((2 * n + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     stream, ws, 2 * n);
  if (items > 0) {
    const bool rope = a.rope_cos != nullptr;
    if (bf16 && !rope)
      launch_calib_d<true, false>(a, (unsigned)items, ws, stream);
    else if (!rope)
      launch_calib_d<false, false>(a, (unsigned)items, ws, stream);
    else if (bf16)
      launch_calib_d<true, true>(a, (unsigned)items, ws, stream);
    else
      launch_calib_d<false, true>(a, (unsigned)items, ws, stream);
  }
  hipLaunchKernelGGL(calib_finish_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     stream, ws, a.smooth, n, a.alpha);
  return hipGetLastError();
}

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
  const bool rope = a.rope_cos != nullptr;
  if (bf16 && !rope)
    launch_d<true, false>(a, (unsigned)total, stream);
  else if (!rope)
    launch_d<false, false>(a, (unsigned)total, stream);
  else if (bf16)
    launch_d<true, true>(a, (unsigned)total, stream);
  else
    launch_d<false, true>(a, (unsigned)total, stream);
  return hipGetLastError();
}

}  // namespace hifa4
