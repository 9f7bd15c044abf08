// attn_bf16.hip -- bf16 FlashAttention forward for gfx950: the accuracy and
// latency baseline ("HiFA4: Training-Free 4-bit FlashAttention on Ascend HIF4
// NPUs for LLM Inference", Abstract, compares the 4-bit operator against bf16
// FlashAttention).  bf16 MFMA products, fp32 online softmax, the normaliser
// summed on the vector ALU from the unrounded P.
//
// Same skeleton as the MXFP4 kernel: S^T = K Q^T on v_mfma_f32_32x32x16_bf16
// with the K rows loaded in a permuted order so that each lane's accumulator
// registers already hold the keys of its P V operand (K = 16 keys per MFMA:
// lane (q, h) needs keys 16u + 8h .. + 7 of MFMA u).  V is staged in LDS
// transposed (channel-major) so its A operand is one 16-byte LDS read.  Tiles
// are double-buffered: the next tile is loaded into registers while the
// current one is computed, then written to the other LDS buffer (V transposed
// four keys at a time, one 8-byte LDS write per channel).
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace hifa4 {
namespace {

constexpr int kBN = 64;
constexpr int kBR = 128;
constexpr float kLn2 = 0.6931471805599453f;

// Two fp32 to a packed bf16 pair with the hardware's round-to-nearest-even
// convert (one gfx950 instruction for both).
__device__ __forceinline__ uint32_t pack_bf16x2(float x, float y) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const f2 v = {x, y};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
}

// Key (within the 64-key step) loaded as A row m of 32-key tile t.
__device__ __forceinline__ int perm_row_bf16(int t, int m) {
  const int j = m >> 3, hh = (m >> 2) & 1, i = m & 3;
  return 32 * t + 16 * (j >> 1) + 8 * hh + 4 * (j & 1) + i;
}

template <int D, bool kCausal>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(Bf16AttnArgs a) {
  constexpr int NJ = D / 16;     // QK MFMAs per 32-key tile
  constexpr int NC = D / 32;     // channel tiles
  constexpr int VT = kBN + 8;    // padded key stride of the transposed V tile (elements)
  // K rows padded by 16 bytes: the 16 lanes of one LDS read phase take 16 different
  // rows at one column, which a power-of-two row stride would put in the same banks
  constexpr int KS = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][kBN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t lds_vt[2][D * VT];
  // per thread and tile: KL 16-byte K chunks, VL groups of (4 keys, 8 channels)
  constexpr int KL = kBN * D / 8 / 256;
  constexpr int VITEMS = (kBN / 4) * (D / 8);
  constexpr int VL = (VITEMS + 255) / 256;
  static_assert(KL >= 1 && KL * 256 == kBN * D / 8, "K tile must split evenly over the workgroup");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, n = lane & 31;
  const int G = a.Hq / a.Hkv;
  const int n_kv = a.B * a.Hkv;
  const int n_qt = (a.Sq + kBR - 1) / kBR;
  int wi = blockIdx.x;
  const int kv = wi % n_kv;
  wi /= n_kv;
  const int hg = wi % G;
  const int qt = n_qt - 1 - wi / G;
  const int b = kv / a.Hkv, g = kv % a.Hkv;
  const int hq = g * G + hg;
  const int L = a.Sk;
  const int64_t bhq = (int64_t)b * a.Hq + hq;
  const int64_t bkv = (int64_t)b * a.Hkv + g;
  const int q_wave0 = qt * kBR + wave * 32;
  const int q = q_wave0 + n;

  v8s qa[NJ];
  if (q < a.Sq) {
    const uint16_t* qr = a.q + (bhq * a.Sq + q) * D;
#pragma unroll
    for (int j = 0; j < NJ; j++) {
      uint4 w = *reinterpret_cast<const uint4*>(qr + 16 * j + 8 * h);
      __builtin_memcpy(&qa[j], &w, 16);
    }
  } else {
#pragma unroll
    for (int j = 0; j < NJ; j++) qa[j] = v8s{};
  }

  int kv_end = L, wave_end = L, wave_full = L;
  if (kCausal) {
    const int last_q = min(a.Sq, (qt + 1) * kBR) - 1;
    kv_end = max(0, min(L, last_q + L - a.Sq + 1));
    const int wl = min(a.Sq, q_wave0 + 32) - 1;
    wave_end = max(0, min(L, wl + L - a.Sq + 1));
    wave_full = max(0, min(L, q_wave0 + L - a.Sq + 1));
  }
  if (q_wave0 >= a.Sq) wave_end = 0;
  const int n_tiles = (kv_end + kBN - 1) / kBN;
  const int row_lim = kCausal ? min(L, q + L - a.Sq + 1) : L;
  const float c = a.sm_log2;

  float m_run = -INFINITY, l_run = 0.0f;
  v16f acc[NC];
#pragma unroll
  for (int cc = 0; cc < NC; cc++) acc[cc] = v16f{};

  // tile loads into registers (keys past L read as zeros) and their LDS stores
  uint4 kr[KL], vr[VL][4];
  auto load_tile = [&](int n0) {
#pragma unroll
    for (int i = 0; i < KL; i++) {
      const int ci = tid + 256 * i;
      const int row = ci / (D / 8), off = (ci % (D / 8)) * 8;
      kr[i] = n0 + row < L
                  ? *reinterpret_cast<const uint4*>(a.k + (bkv * a.cap + n0 + row) * D + off)
                  : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < VL; i++) {
      const int ci = tid + 256 * i;
      const int k4 = ci % (kBN / 4), cg = (ci / (kBN / 4)) * 8;
#pragma unroll
      for (int kk = 0; kk < 4; kk++) {
        const int key = 4 * k4 + kk;
        vr[i][kk] = ci < VITEMS && n0 + key < L
                        ? *reinterpret_cast<const uint4*>(a.v + (bkv * a.cap + n0 + key) * D + cg)
                        : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KL; i++) {
      const int ci = tid + 256 * i;
      const int row = ci / (D / 8), off = (ci % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(lds_k[buf] + row * KS + off) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < VL; i++) {
      const int ci = tid + 256 * i;
      if (ci >= VITEMS) break;
      const int k4 = ci % (kBN / 4), cg = (ci / (kBN / 4)) * 8;
      const uint32_t wk[4][4] = {{vr[i][0].x, vr[i][0].y, vr[i][0].z, vr[i][0].w},
                                 {vr[i][1].x, vr[i][1].y, vr[i][1].z, vr[i][1].w},
                                 {vr[i][2].x, vr[i][2].y, vr[i][2].z, vr[i][2].w},
                                 {vr[i][3].x, vr[i][3].y, vr[i][3].z, vr[i][3].w}};
      // channel c of keys 4 k4 .. 4 k4 + 3: one 8-byte write
#pragma unroll
      for (int c2 = 0; c2 < 4; c2++) {
        const uint32_t w0 = wk[0][c2], w1 = wk[1][c2], w2 = wk[2][c2], w3 = wk[3][c2];
        // low halves: channel cg + 2 c2, high halves: channel cg + 2 c2 + 1
        const uint2 lo = make_uint2((w0 & 0xFFFFu) | (w1 << 16), (w2 & 0xFFFFu) | (w3 << 16));
        const uint2 hi = make_uint2((w0 >> 16) | (w1 & 0xFFFF0000u), (w2 >> 16) | (w3 & 0xFFFF0000u));
        *reinterpret_cast<uint2*>(lds_vt[buf] + (cg + 2 * c2) * VT + 4 * k4) = lo;
        *reinterpret_cast<uint2*>(lds_vt[buf] + (cg + 2 * c2 + 1) * VT + 4 * k4) = hi;
      }
    }
  };
  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int kt = 0; kt < n_tiles; kt++) {
    const int n0 = kt * kBN;
    const int buf = kt & 1;
    const bool more = kt + 1 < n_tiles;  // uniform
    if (more) load_tile(n0 + kBN);
    const uint16_t* lk = lds_k[buf];
    const uint16_t* lv = lds_vt[buf];
    if (n0 < wave_end) {

    v16f s0 = v16f{}, s1 = v16f{};
    const int r0 = perm_row_bf16(0, n), r1 = perm_row_bf16(1, n);
#pragma unroll
    for (int j = 0; j < NJ; j++) {
      v8s k0, k1;
      uint4 w0 = *reinterpret_cast<const uint4*>(lk + r0 * KS + 16 * j + 8 * h);
      uint4 w1 = *reinterpret_cast<const uint4*>(lk + r1 * KS + 16 * j + 8 * h);
      __builtin_memcpy(&k0, &w0, 16);
      __builtin_memcpy(&k1, &w1, 16);
      s0 = mfma_bf16_32x32x16(k0, qa[j], s0);
      s1 = mfma_bf16_32x32x16(k1, qa[j], s1);
    }
    // lane (q, h): tile t register r holds key 32t + 16*(r/8) + 8h + r%8
    float s[32];
#pragma unroll
    for (int r = 0; r < 16; r++) {
      s[r] = s0[r];
      s[16 + r] = s1[r];
    }
    if (n0 + kBN > wave_full) {
#pragma unroll
      for (int k = 0; k < 32; k++) {
        const int key = n0 + 32 * (k >> 4) + 16 * ((k >> 3) & 1) + 8 * h + (k & 7);
        if (key >= row_lim) s[k] = -INFINITY;
      }
    }
    float bm = s[0];
#pragma unroll
    for (int k = 1; k < 32; k++) bm = fmaxf(bm, s[k]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm),
                                                     false, false);
    const float rmc = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c;
    // lazy rescale (same rule as the MXFP4 kernel; exact attention is frame-free)
    const float m_new = rmc > m_run + a.tau ? rmc : m_run;
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float p[32];
    float ps = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; k++) {
      p[k] = __builtin_amdgcn_exp2f(fmaf(s[k], c, -m_use));
      ps += p[k];
    }
    {
      const auto pw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ps), __float_as_uint(ps),
                                                       false, false);
      ps = __uint_as_float(pw[0]) + __uint_as_float(pw[1]);
    }
    l_run = alpha * l_run + ps;
    m_run = m_new;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int cc = 0; cc < NC; cc++) acc[cc] *= alpha;
    }
    // P V: 4 MFMAs of 16 keys; MFMA u = 2t + j2 takes registers 8*j2 .. +7 of tile t
#pragma unroll
    for (int u = 0; u < 4; u++) {
      uint32_t pw[4];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int k = 16 * (u >> 1) + 8 * (u & 1) + 2 * i;
        pw[i] = pack_bf16x2(p[k], p[k + 1]);
      }
      v8s pb;
      __builtin_memcpy(&pb, pw, 16);
#pragma unroll
      for (int cc = 0; cc < NC; cc++) {
        v8s va;
        uint4 w = *reinterpret_cast<const uint4*>(lv + (32 * cc + n) * VT + 16 * u + 8 * h);
        __builtin_memcpy(&va, &w, 16);
        acc[cc] = mfma_bf16_32x32x16(va, pb, acc[cc]);
      }
    }
    }  // n0 < wave_end
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (q < a.Sq) {
    const int64_t row = bhq * a.Sq + q;
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
#pragma unroll
    for (int cc = 0; cc < NC; cc++)
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        const int ch = 32 * cc + 8 * g4 + 4 * h;
        *reinterpret_cast<uint2*>(a.out + row * D + ch) =
            make_uint2(pack_bf16x2(acc[cc][4 * g4] * inv, acc[cc][4 * g4 + 1] * inv),
                       pack_bf16x2(acc[cc][4 * g4 + 2] * inv, acc[cc][4 * g4 + 3] * inv));
      }
    if (a.lse && h == 0) a.lse[row] = l_run > 0.0f ? m_run * kLn2 + logf(l_run) : -INFINITY;
  }
}

template <int D>
hipError_t launch_d(const Bf16AttnArgs& a, hipStream_t stream) {
  const int n_qt = (a.Sq + kBR - 1) / kBR;
  const int64_t grid = (int64_t)n_qt * a.B * a.Hq;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (a.causal)
    hipLaunchKernelGGL((attn_bf16_kernel<D, true>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, false>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_prefill_bf16(const Bf16AttnArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 64: return launch_d<64>(a, stream);
    case 128: return launch_d<128>(a, stream);
    case 256: return launch_d<256>(a, stream);
  }
  return hipErrorNotSupported;
}

}  // namespace hifa4
