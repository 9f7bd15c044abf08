// attn_bf16.hip -- bf16 FlashAttention forward for gfx950: the accuracy and
// latency baseline ("HiFA4: Training-Free 4-bit FlashAttention on Ascend HIF4
// NPUs for LLM Inference", Abstract, compares the 4-bit operator against bf16
// FlashAttention).  bf16 MFMA products, fp32 online softmax, the normaliser
// summed on the vector ALU from the unrounded P.
//
// Same skeleton as the MXFP4 kernel: S^T = K Q^T on v_mfma_f32_32x32x16_bf16
// with the K rows staged in a permuted order so that each lane's accumulator
// registers already hold the keys of its P V operand (K = 16 keys per MFMA:
// lane (q, h) needs keys 16u + 8h .. + 7 of MFMA u).  K and V tiles go from
// memory straight into LDS (buffer loads with the LDS destination) through
// two-stage rings; V keeps its row-major layout and its operand (8 keys of
// one channel per lane) is read with the gfx950 LDS transpose read
// (ds_read_b64_tr_b16).  K runs one tile ahead of V: step kt loads K tile
// kt+2 and V tile kt+1, and, at raised wave priority, runs the Q K^T MFMAs of
// tile kt+1 interleaved with the softmax of tile kt, then the P V MFMAs of
// tile kt.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "launch.hpp"
#include "lds_dma.hpp"

namespace hifa4 {
namespace {

typedef short v4s __attribute__((ext_vector_type(4)));

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

// Key (within the 64-key step) staged as A row m of 32-key tile t.
__device__ __forceinline__ int perm_row_bf16(int t, int m) {
  const int j = m >> 3, hh = (m >> 2) & 1, i = m & 3;
  return 32 * t + 16 * (j >> 1) + 8 * hh + 4 * (j & 1) + i;
}

// LDS stage layouts (one stage = one 64-key tile of K or of V, D bf16 per key).
// Rows of RB = 2D bytes, NCH 16-byte chunks each; chunk c of row R sits in slot
// c ^ swizzle(R), so that the operand reads of one LDS pass fall in distinct
// banks (64 banks of 4 bytes):
//  - K: row R = 32t + m holds key perm_row_bf16(t, m); a Q K^T read takes rows
//    m = 0..15 at one chunk: the swizzle spreads them over the 16 bank groups;
//  - V: row R holds key R; a transpose read takes rows r..r+3 (r % 4 == 0) at
//    chunks 4cc..4cc+3: the swizzle 4 * (R % 4) puts the 16 in distinct groups.
template <int D>
struct Bf16Stage {
  static constexpr int RB = 2 * D;
  static constexpr int NCH = RB / 16;
  static constexpr int BYTES = kBN * RB;
  static constexpr int LOADS = BYTES / 1024 / 4;  // 1 KB loads per wave (4 waves)
  static_assert(LOADS >= 1 && LOADS * 4096 == BYTES, "a stage splits into 1 KB loads per wave");
};
template <int D>
__device__ __forceinline__ int k_swz_bf16(int R) {
  return D == 64 ? (R >> 1) & 7 : R & 15;
}
template <int D>
__device__ __forceinline__ int v_swz_bf16(int R) {
  return D == 64 ? 4 * ((R >> 1) & 1) : 4 * (R & 3);
}

template <int D, bool kCausal>
__global__ __launch_bounds__(256, D == 256 ? 1 : 2) void attn_bf16_kernel(Bf16AttnArgs a) {
  using T = Bf16Stage<D>;
  constexpr int NJ = D / 16;     // QK MFMAs per 32-key tile
  constexpr int NC = D / 32;     // channel tiles
  constexpr int RB = T::RB;
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[2 * T::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[2 * T::BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  // Staging: one descriptor per (batch, KV head) over its L valid keys (rows
  // past them read zeros); lane i of load ii of this wave fills LDS slot
  // p = (wave * LOADS + ii) * 64 + i of a stage, i.e. row p / NCH, slot p % NCH.
  const v4i kdesc = buffer_desc(a.k + bkv * a.cap * D, (uint32_t)L * RB);
  const v4i vdesc = buffer_desc(a.v + bkv * a.cap * D, (uint32_t)L * RB);
  uint32_t koff_src[T::LOADS], voff_src[T::LOADS];
#pragma unroll
  for (int ii = 0; ii < T::LOADS; ii++) {
    const int p = (wave * T::LOADS + ii) * 64 + lane;
    const int R = p / T::NCH, sl = p % T::NCH;
    koff_src[ii] = (uint32_t)(perm_row_bf16(R >> 5, R & 31) * RB + ((sl ^ k_swz_bf16<D>(R)) * 16));
    voff_src[ii] = (uint32_t)(R * RB + ((sl ^ v_swz_bf16<D>(R)) * 16));
  }
  const uint32_t kdst = lds_addr(lds_k) + wave * T::LOADS * 1024;
  const uint32_t vdst = lds_addr(lds_v) + wave * T::LOADS * 1024;
  auto issue_k = [&](auto stage, int tile) {
    constexpr int ST = decltype(stage)::value;
    const int so = tile < n_tiles ? tile * kBN * RB : 0x7FFFFFF0;
#pragma unroll
    for (int ii = 0; ii < T::LOADS; ii++) {
      switch (ii) {  // the LDS immediate must be a constant
#define HIFA4_BF16_K(I) case I: if constexpr (I < T::LOADS) load_lds16<ST * T::BYTES + I * 1024>(kdesc, koff_src[I], so, kdst); break;
        HIFA4_BF16_K(0) HIFA4_BF16_K(1) HIFA4_BF16_K(2) HIFA4_BF16_K(3)
        HIFA4_BF16_K(4) HIFA4_BF16_K(5) HIFA4_BF16_K(6) HIFA4_BF16_K(7)
#undef HIFA4_BF16_K
      }
    }
  };
  auto issue_v = [&](auto stage, int tile) {
    constexpr int ST = decltype(stage)::value;
    const int so = tile < n_tiles ? tile * kBN * RB : 0x7FFFFFF0;
#pragma unroll
    for (int ii = 0; ii < T::LOADS; ii++) {
      switch (ii) {
#define HIFA4_BF16_V(I) case I: if constexpr (I < T::LOADS) load_lds16<ST * T::BYTES + I * 1024>(vdesc, voff_src[I], so, vdst); break;
        HIFA4_BF16_V(0) HIFA4_BF16_V(1) HIFA4_BF16_V(2) HIFA4_BF16_V(3)
        HIFA4_BF16_V(4) HIFA4_BF16_V(5) HIFA4_BF16_V(6) HIFA4_BF16_V(7)
#undef HIFA4_BF16_V
      }
    }
  };
  static_assert(T::LOADS <= 8, "at most eight loads per wave and tile");

  // Q operand (B of S^T = K Q^T): query q, elements 16j + 8h .. + 7
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

  // The lane's K operand offsets in a stage: row n (tile 0; tile 1 adds 32
  // rows, whose swizzle is the same), chunk 2j + h.
  uint32_t koff[NJ];
#pragma unroll
  for (int j = 0; j < NJ; j++) koff[j] = (uint32_t)(n * RB + (((2 * j + h) ^ k_swz_bf16<D>(n)) * 16));
  // The lane's V transpose-read offsets: in its 16-lane group gq = lane / 16
  // the lane (4i + a4) points at key 8 (gq / 2) + i (plus 16u + 4r per read)
  // and channels 32cc + 16 (gq % 2) + 4 a4 .. + 3; the read returns channel
  // 32cc + n of keys 16u + 8h + 4r .. + 3 to lane (n, h).
  uint32_t voff[NC];
  {
    const int gq = lane >> 4, jl = lane & 15, i4 = jl >> 2, a4 = jl & 3;
    const int R = 8 * (gq >> 1) + i4;
#pragma unroll
    for (int cc = 0; cc < NC; cc++) {
      const int byte = 2 * (32 * cc + 16 * (gq & 1) + 4 * a4);  // within the row
      voff[cc] = (uint32_t)(R * RB + (((byte >> 4) ^ v_swz_bf16<D>(R)) << 4) + (byte & 15));
    }
  }

  float m_run = -INFINITY, l_run = 0.0f;
  v16f acc[NC];
#pragma unroll
  for (int cc = 0; cc < NC; cc++) acc[cc] = v16f{};

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // S^T = K Q^T of the tile in K stage ks
  auto qk = [&](int ks_bytes, v16f& s0, v16f& s1) {
    const uint8_t* lk = lds_k + ks_bytes;
    s0 = v16f{};
    s1 = v16f{};
#pragma unroll
    for (int j = 0; j < NJ; j++) {
      v8s k0, k1;
      const uint4 w0 = *reinterpret_cast<const uint4*>(lk + koff[j]);
      const uint4 w1 = *reinterpret_cast<const uint4*>(lk + 32 * RB + koff[j]);
      __builtin_memcpy(&k0, &w0, 16);
      __builtin_memcpy(&k1, &w1, 16);
      s0 = mfma_bf16_32x32x16(k0, qa[j], s0);
      s1 = mfma_bf16_32x32x16(k1, qa[j], s1);
    }
  };

  // prologue: K tiles 0, 1 and V tile 0
  issue_k(S0{}, 0);
  issue_v(S0{}, 0);
  issue_k(S1{}, 1);
  HIFA4_WAIT_VMCNT(0);
  __syncthreads();
  // a wave whose rows see no key never computes (sa0, sa1): zeros, then masked
  v16f sa0 = v16f{}, sa1 = v16f{}, sb0, sb1;
  if (n_tiles > 0) qk(0, sa0, sa1);
  // step 0 refills K stage 0: every wave's reads of it come first
  __syncthreads();

  // One step on tile kt (K and V stage kt % 2 = ST), scores in (c0, c1): loads
  // of K tile kt+2 (into K stage ST, whose tile kt was read by step kt-1) and
  // V tile kt+1 (into V stage ST ^ 1, whose tile kt-1 step kt-1 read); at wave
  // priority 1 the softmax of tile kt interleaved with the Q K^T MFMAs of tile
  // kt+1 (K stage ST ^ 1, into (n0r, n1r)), then the P V MFMAs of tile kt;
  // wait for this step's loads; barrier.  A wave whose rows see no key of tile
  // kt masks all its scores (P = 0, the running max stays); the products of a
  // tile past the last read finite stale LDS and are discarded.
  auto step = [&](auto stage, int kt, v16f& c0, v16f& c1, v16f& n0r, v16f& n1r) {
    constexpr int ST = decltype(stage)::value;
    using SN = std::integral_constant<int, ST ^ 1>;
    const int n0 = kt * kBN;
    issue_k(stage, kt + 2);
    issue_v(SN{}, kt + 1);
    float s[32];
#pragma unroll
    for (int r = 0; r < 16; r++) {
      s[r] = c0[r];
      s[16 + r] = c1[r];
    }
    // lane (q, h): tile t register r holds key 32t + 16*(r/8) + 8h + r%8
    if (n0 >= wave_end || n0 + kBN > wave_full) {
      const int lim = n0 < wave_end ? row_lim : 0;
#pragma unroll
      for (int k = 0; k < 32; k++) {
        const int key = n0 + 32 * (k >> 4) + 16 * ((k >> 3) & 1) + 8 * h + (k & 7);
        if (key >= lim) s[k] = -INFINITY;
      }
    }
    // max3 tree over the 32 scores, then the partner half's
    float u[11];
#pragma unroll
    for (int i = 0; i < 10; i++)
      u[i] = __builtin_elementwise_maximum(__builtin_elementwise_maximum(s[3 * i], s[3 * i + 1]),
                                           s[3 * i + 2]);
    u[10] = __builtin_elementwise_maximum(s[30], s[31]);
    float bm = u[0];
#pragma unroll
    for (int i = 1; i < 11; i++) bm = __builtin_elementwise_maximum(bm, u[i]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm),
                                                     false, false);
    const float rmc =
        __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c;
    // lazy rescale (same rule as the MXFP4 kernel; exact attention is frame-free)
    const float m_new = rmc > m_run + a.tau ? rmc : m_run;
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    asm volatile("" : "+v"(qa[0][0]) : "v"(m_use));
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    qk((ST ^ 1) * T::BYTES, n0r, n1r);
#pragma unroll
    for (int k = 0; k < 32; k++) s[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[k], c, -m_use));
    // row sum as a tree
    float t16[16];
#pragma unroll
    for (int k = 0; k < 16; k++) t16[k] = s[2 * k] + s[2 * k + 1];
#pragma unroll
    for (int k = 0; k < 8; k++) t16[k] = t16[2 * k] + t16[2 * k + 1];
#pragma unroll
    for (int k = 0; k < 4; k++) t16[k] = t16[2 * k] + t16[2 * k + 1];
    float ps = (t16[0] + t16[1]) + (t16[2] + t16[3]);
    v8s pb[4];
#pragma unroll
    for (int uu = 0; uu < 4; uu++) {
      uint32_t pw[4];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int k = 16 * (uu >> 1) + 8 * (uu & 1) + 2 * i;
        pw[i] = pack_bf16x2(s[k], s[k + 1]);
      }
      __builtin_memcpy(&pb[uu], pw, 16);
    }
    // the K operand reads two MFMAs ahead; each Q K^T MFMA followed by a few
    // vector instructions of the softmax (4 at d = 128: 156.7 -> 144.7 us on the
    // Qwen3 shape; 8 at d = 256)
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < 2 * NJ; i++) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, D == 64 ? 12 : (D == 128 ? 4 : 8), 0);
    }
    __builtin_amdgcn_sched_barrier(0);
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
    // P V: MFMA (u, cc) takes keys 16u .. 16u + 15 of channel tile cc; the
    // lane's operand is two transpose reads of 4 keys each (keys 16u + 8h + 4r)
    typedef __attribute__((address_space(3))) v4s* lds_v4s;
    const uint8_t* lv = lds_v + ST * T::BYTES;
#pragma unroll
    for (int uu = 0; uu < 4; uu++) {
#pragma unroll
      for (int cc = 0; cc < NC; cc++) {
        const uint8_t* p0 = lv + voff[cc] + (16 * uu) * RB;
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4s)(__attribute__((address_space(3))) uint8_t*)p0);
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4s)(__attribute__((address_space(3))) uint8_t*)(p0 + 4 * RB));
        const v8s va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[cc] = mfma_bf16_32x32x16(va, pb[uu], acc[cc]);
      }
    }
    // the V operand reads two MFMAs ahead
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
    for (int i = 0; i < 4 * NC; i++) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    }
    // the next tile's scores may not sink past the barrier into the next step
    asm volatile("" : "+v"(n0r[0]), "+v"(n1r[0]));
    __builtin_amdgcn_s_setprio(0);
    HIFA4_WAIT_VMCNT(0);
    __syncthreads();
  };
  for (int kt = 0; kt < n_tiles; kt += 2) {
    step(S0{}, kt, sa0, sa1, sb0, sb1);
    if (kt + 1 >= n_tiles) break;
    step(S1{}, kt + 1, sb0, sb1, sa0, sa1);
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
