// attn_mxfp4.hip -- fused MXFP4 FlashAttention for gfx950: prefill and
// split-K decode with a log-sum-exp merge.
//
// Method: "HiFA4: Training-Free 4-bit FlashAttention on Ascend HIF4 NPUs for
// LLM Inference", Abstract:
//   - Q K^T and P V are both 4-bit block-scaled products: here the gfx950
//     scaled-FP4 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4), E2M1 operands with
//     E8M0 scales per 32 elements fed straight into the instruction;
//   - the online-softmax state (running max m, normaliser l) stays in higher
//     precision than the operands (fp32 here);
//   - P-Reordering: P = exp(S - m_new) is quantised to MXFP4 in registers and
//     the normaliser is summed from that same P_hat; the sum is fused into the
//     P V product by appending an all-ones column to V (an extra 32-row MFMA
//     tile whose row 0 is E2M1 1.0 with scale 2^0), so l comes out of the
//     matrix core next to P_hat V.
//
// Layouts (see include/hifa4.h): Q / K rows hold d/2 code bytes and d/32
// scale bytes; V is key-blocked, every channel's 32 tokens contiguous in 16
// bytes, which is exactly one lane's P V operand.
//
// Register layouts of the 32x32x64 MFMA (checked by the probe tests):
// lane l supplies row / column l % 32 and the 32-element K block l / 32; the
// accumulator register r of lane l holds D[8*(r/4) + 4*(l/32) + r%4][l % 32].
//
// S is computed transposed (S^T = K Q^T), so a lane owns one query and 16
// keys per 32-key tile.  The K rows of the A operand are loaded in the
// permuted order perm_row(), chosen so that after the two 32-key MFMAs of a
// 64-key step, lane (q, h) holds exactly keys 32h .. 32h+31 of that step, in
// order, in registers (tile t, register r) -> key 32h + 16t + r.  That is the
// B-operand layout of the P V MFMA (K = 64 keys, block h), so P goes from the
// accumulator to the next MFMA with no cross-lane traffic: its block max is
// an in-lane max, its 32 values are packed by 16 v_cvt_scalef32_pk_fp4_f32.
// The row max over a step needs one exchange between lanes l and l ^ 32.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

// Products and sums are rounded separately unless fmaf is spelled out: the
// softmax relies on fl(S * c) being the same value in the max and in the
// block-scale exponent.
#pragma clang fp contract(off)

namespace hifa4 {

namespace {

constexpr int kBN = 64;            // keys per online-softmax step (the P frame tile)
constexpr int kWaves = 4;          // waves per workgroup
constexpr int kBR = 32 * kWaves;   // queries per prefill workgroup
constexpr int kDecodeChunk = 512;  // tokens per decode wave (fresh state), default
constexpr float kLn2 = 0.6931471805599453f;

// Row of the 64-key step that A-operand row m of 32-key tile t loads.
__device__ __forceinline__ int perm_row(int t, int m) {
  return 32 * ((m >> 2) & 1) + 16 * t + 4 * (m >> 3) + (m & 3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// One online-softmax step on the 32 scores a lane holds for its query
// (already masked with -inf).  Updates m_run, rescales the accumulators and
// returns the packed P operand plus its E8M0 byte.
struct SoftmaxStep {
  uint4 p_codes;
  int p_scale;
  float alpha;
};

//
// Lazy rescale: the running max m moves to the tile's row max only when that
// exceeds m by more than tau (log2 units); otherwise the frame is kept and P
// may reach 2^tau.  tau = 0 is the FlashAttention-2 frame (P <= 1).  Exact
// attention does not depend on the frame; P_hat does, so tau is part of the
// operator's definition (the oracle takes the same value).
//
// The running max and the block scale of P are taken from the *rounded*
// products fl(S * c): the row max is max_k fl(S_k * c) (rounding is monotone,
// so this is fl(max_k S_k * c)), and the block maximum of P is
// exp2(fl(bm * c) - m_new), which is exactly 1 for the block holding the row
// max when the frame moves to it, as in exact arithmetic.  (Taking it from the
// fused fma(S, c, -m) instead would see the product's rounding error: the row
// max could come out as 1 - 2^-24, dropping that block's E8M0 exponent by one
// and saturating its largest P to 0.75.)  The P elements themselves use the
// fused form; the row max then lands within an ulp of 1 and rounds to 4.0.
//
// The row max needs the partner lane l ^ 32 (the other 32 keys of the step):
// v_permlane32_swap exchanges the two halves of the wave in one VALU op, and
// the max of its two results is max(own, partner) in every lane.
__device__ __forceinline__ float fmax_(float a, float b) {
  // IEEE maximum (v_maximum3_f32): no NaN-quieting of the operands needed
  return __builtin_elementwise_maximum(a, b);
}

__device__ __forceinline__ float max_with_half_swap(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmax_(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Softmax step on the lane's 32 scores held in the two QK accumulators (tile
// t, register r <-> key 32h + 16t + r), in place: the scores are replaced by
// P before packing, so no copies of the accumulators are made.  Masked
// scores are -inf on entry.
//
// `pk` is the previous step's packed P: every byte of it is overwritten, it
// only gives the partial-write converts a register to start from.
__device__ __forceinline__ SoftmaxStep softmax_step(v16f& s0, v16f& s1, float& m_run, float c,
                                                    float tau, uint4& pk) {
  float ma = s0[0], mb = s1[0];
#pragma unroll
  for (int r = 1; r < 16; r++) {
    ma = fmax_(ma, s0[r]);
    mb = fmax_(mb, s1[r]);
  }
  const float bm = fmax_(ma, mb);
  const float bmc = bm * c;  // contraction is off in this file: a rounded product
  const float rmc = max_with_half_swap(bmc);
  const float m_new = rmc > m_run + tau ? rmc : m_run;
  const float m_use = m_new == -INFINITY ? 0.0f : m_new;
  SoftmaxStep st;
  st.alpha = fast_exp2(m_run - m_use);
#pragma unroll
  for (int r = 0; r < 16; r++) {
    s0[r] = fast_exp2(__builtin_fmaf(s0[r], c, -m_use));
    s1[r] = fast_exp2(__builtin_fmaf(s1[r], c, -m_use));
  }
  const float pmax = fast_exp2(bmc - m_use);
  const uint32_t sb = e8m0_from_amax(pmax);
  st.p_scale = (int)sb;
  const float scale = e8m0_to_float(sb);
  uint32_t w[4] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const v16f& src = q < 2 ? s0 : s1;
    const int o = 8 * (q & 1);
    uint32_t x = w[q];
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, src[o + 0], src[o + 1], scale, 0);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, src[o + 2], src[o + 3], scale, 1);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, src[o + 4], src[o + 5], scale, 2);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, src[o + 6], src[o + 7], scale, 3);
    w[q] = x;
  }
  st.p_codes = make_uint4(w[0], w[1], w[2], w[3]);
  pk = st.p_codes;
  m_run = m_new;
  return st;
}

// Mask keys >= lim (key of element (t, r) is kb + 16t + r) with -inf.
__device__ __forceinline__ void mask_scores(v16f& s0, v16f& s1, int kb, int lim) {
  const int rem = lim - kb;  // elements r < rem stay
#pragma unroll
  for (int r = 0; r < 16; r++) {
    if (r >= rem) s0[r] = -INFINITY;
    if (16 + r >= rem) s1[r] = -INFINITY;
  }
}

template <int NC>
__device__ __forceinline__ void write_out(const AttnArgs& a, int64_t row, int h, const v16f (&acc)[NC],
                                          float inv) {
  constexpr int D = NC * 32;
#pragma unroll
  for (int c = 0; c < NC; c++) {
#pragma unroll
    for (int g4 = 0; g4 < 4; g4++) {
      const int ch = 32 * c + 8 * g4 + 4 * h;
      uint32_t u[4];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float v = acc[c][4 * g4 + i] * inv;
        u[i] = a.out_fp16 ? float_to_half_bits(v) : float_to_bf16_bits(v);
      }
      uint2 w = make_uint2(u[0] | (u[1] << 16), u[2] | (u[3] << 16));
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + row * D + ch) = w;
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill: one workgroup = 128 queries of one (batch, query head); 4 waves of
// 32 queries share 64-key K / V tiles staged in LDS.
//
// Software pipeline.  Step kt of a wave issues the Q K^T MFMAs of tile kt+1
// first, then runs the softmax of tile kt (whose scores came out of the
// previous step) and its P V MFMAs: the matrix core computes the next scores
// while the vector ALU does the exponentials and FP4 conversions.  K is
// therefore staged one tile ahead of V: during step kt the LDS holds K of
// tile kt+1 and V of tile kt, and the bytes of K tile kt+2 / V tile kt+1 are
// in flight into registers; they are written to the free buffers at the end
// of the step and one barrier per step publishes them.
//
// K rows are stored in LDS in the order the MFMA A operand reads them (row
// 32t + n of a buffer holds key perm_row(t, n)) with a padded stride of
// d/2 + 16 bytes, so the 16-byte reads of 8 neighbouring lanes fall in
// distinct bank groups.
// ---------------------------------------------------------------------------
template <int D>
struct PrefillTile {
  static constexpr int DB = D / 2;               // code bytes per K row
  static constexpr int DS = D / 32;              // scale bytes per K row
  static constexpr int RS = DB + 16;             // padded LDS stride of a K row
  static constexpr int KC = kBN * DB / 16;       // 16-byte K code chunks per tile
  static constexpr int VC = 2 * D;               // 16-byte V code chunks per tile
  static constexpr int KC_T = (KC + 255) / 256;  // per thread
  static constexpr int VC_T = (VC + 255) / 256;
  static constexpr int VS_W = 2 * D / 4;         // 4-byte V scale words per tile
  static constexpr int LDS_K = kBN * RS + kBN * DS;   // codes + scales of one K tile
  static constexpr int LDS_V = VC * 16 + 2 * D;       // codes + scales of one V tile
};

// LDS row of key r in the read order of the QK A operand.
__device__ __forceinline__ int k_lds_row(int r) {
  return 32 * ((r >> 4) & 1) + 8 * ((r >> 2) & 3) + 4 * (r >> 5) + (r & 3);
}

template <int D>
struct KRegs {
  uint4 kc[PrefillTile<D>::KC_T];
  uint2 ks;  // DS scale bytes of one K row (threads < 64)
};

template <int D>
struct VRegs {
  uint4 vc[PrefillTile<D>::VC_T];
  uint32_t vs;  // one 4-byte word of V scales
};

// Raw buffer resource (stride 0) over `bytes` bytes from `base`: the
// hardware range check turns every load at or past `bytes` into zeros.  The
// third descriptor word is the gfx9-family default (32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Global loads of a 64-key tile starting at n0.  A tile's K codes, K scales,
// V codes and V scales are each one contiguous run of bytes, so thread tid
// loads chunk tid (+ 256 i) of each at a fixed lane offset from a uniform
// tile base.  The buffer resources end at the last valid key (K) / block
// (V): rows and blocks past them read as zeros (E2M1 zeros with the E8M0
// byte 0, i.e. finite), their scores are masked and their P is zero, so
// they never contribute.  No per-lane clamping or 64-bit address math.
template <int D>
__device__ __forceinline__ void load_k(const AttnArgs& a, int64_t bkv, int n0, int L, int tid,
                                       KRegs<D>& r) {
  using T = PrefillTile<D>;
  const int64_t row0 = bkv * a.cap + n0;
  const uint32_t rows = (uint32_t)(L - n0);
  const auto kc = buffer_rsrc(a.k_codes + row0 * T::DB, rows * T::DB);
  const auto ks = buffer_rsrc(a.k_scales + row0 * T::DS, rows * T::DS);
#pragma unroll
  for (int i = 0; i < T::KC_T; i++) {
    const int ci = tid + 256 * i;
    if (ci < T::KC) r.kc[i] = buffer_load16(kc, (uint32_t)ci * 16u);
  }
  if (tid < kBN) {
    const uint32_t off = (uint32_t)tid * T::DS;
    if constexpr (T::DS == 2) {
      r.ks = make_uint2(__builtin_amdgcn_raw_buffer_load_b16(ks, off, 0, 0), 0);
    } else if constexpr (T::DS == 4) {
      r.ks = make_uint2(__builtin_amdgcn_raw_buffer_load_b32(ks, off, 0, 0), 0);
    } else {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(ks, off, 0, 0);
      r.ks = make_uint2(v[0], v[1]);
    }
  }
}

template <int D>
__device__ __forceinline__ void load_v(const AttnArgs& a, int64_t bkv, int n0, int nblk_valid,
                                       int nblk_cap, int tid, VRegs<D>& r) {
  using T = PrefillTile<D>;
  const int b0 = n0 / 32;
  const int64_t blk0 = bkv * nblk_cap + b0;
  const uint32_t blks = (uint32_t)(nblk_valid - b0);
  const auto vc = buffer_rsrc(a.v_codes + blk0 * D * 16, blks * D * 16);
  const auto vs = buffer_rsrc(a.v_scales + blk0 * D, blks * D);
#pragma unroll
  for (int i = 0; i < T::VC_T; i++) {
    const int ci = tid + 256 * i;
    if (ci < T::VC) r.vc[i] = buffer_load16(vc, (uint32_t)ci * 16u);
  }
  if (tid < T::VS_W) r.vs = __builtin_amdgcn_raw_buffer_load_b32(vs, (uint32_t)tid * 4u, 0, 0);
}

template <int D>
__device__ __forceinline__ void store_k(uint8_t* buf, int tid, const KRegs<D>& r) {
  using T = PrefillTile<D>;
  uint8_t* ks = buf + kBN * T::RS;
#pragma unroll
  for (int i = 0; i < T::KC_T; i++) {
    const int ci = tid + 256 * i;
    if (ci < T::KC) {
      const int row = ci / (T::DB / 16), off = (ci % (T::DB / 16)) * 16;
      *reinterpret_cast<uint4*>(buf + k_lds_row(row) * T::RS + off) = r.kc[i];
    }
  }
  if (tid < kBN) {
    uint8_t* dst = ks + k_lds_row(tid) * T::DS;
    if constexpr (T::DS == 2) {
      *reinterpret_cast<uint16_t*>(dst) = (uint16_t)r.ks.x;
    } else if constexpr (T::DS == 4) {
      *reinterpret_cast<uint32_t*>(dst) = r.ks.x;
    } else {
      *reinterpret_cast<uint2*>(dst) = r.ks;
    }
  }
}

template <int D>
__device__ __forceinline__ void store_v(uint8_t* buf, int tid, const VRegs<D>& r) {
  using T = PrefillTile<D>;
#pragma unroll
  for (int i = 0; i < T::VC_T; i++) {
    const int ci = tid + 256 * i;
    if (ci < T::VC) *reinterpret_cast<uint4*>(buf + ci * 16) = r.vc[i];
  }
  if (tid < T::VS_W) *reinterpret_cast<uint32_t*>(buf + T::VC * 16 + tid * 4) = r.vs;
}

// Scale operand of K block (2j + h) of a row whose DS scale bytes start at p:
// the 32-bit word holding it, shifted by 8h so that byte 2*(j%2) is the one.
template <int DS>
__device__ __forceinline__ int k_scale_word(const uint8_t* p, int j, int h) {
  if constexpr (DS == 2) {
    return (int)(*reinterpret_cast<const uint16_t*>(p) >> (8 * h));
  } else {
    return (int)(reinterpret_cast<const uint32_t*>(p)[j >> 1] >> (8 * h));
  }
}

template <int OPSEL>
__device__ __forceinline__ v16f mfma_fp4_sel(const uint4& a, const uint4& b, const v16f& c, int sa,
                                             int sb) {
  v8i A = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  v8i B = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c, kFmtFp4, kFmtFp4, OPSEL, sa,
                                                         OPSEL, sb);
}

// S^T = K Q^T for the two 32-key tiles of a 64-key step held in one K buffer.
template <int D>
__device__ __forceinline__ void qk_step(const uint8_t* kbuf, const uint4 (&qa)[D / 64],
                                        const int (&qsw)[(D / 64 + 1) / 2], int n, int h,
                                        v16f& s0, v16f& s1) {
  using T = PrefillTile<D>;
  constexpr int NJ = D / 64;
  const uint8_t* ks = kbuf + kBN * T::RS;
  s0 = v16f{};
  s1 = v16f{};
#pragma unroll
  for (int j = 0; j < NJ; j++) {
    const uint4 k0 = *reinterpret_cast<const uint4*>(kbuf + n * T::RS + 32 * j + 16 * h);
    const uint4 k1 = *reinterpret_cast<const uint4*>(kbuf + (32 + n) * T::RS + 32 * j + 16 * h);
    const int ks0 = k_scale_word<T::DS>(ks + n * T::DS, j, h);
    const int ks1 = k_scale_word<T::DS>(ks + (32 + n) * T::DS, j, h);
    if (j % 2 == 0) {
      s0 = mfma_fp4_sel<0>(k0, qa[j], s0, ks0, qsw[j / 2]);
      s1 = mfma_fp4_sel<0>(k1, qa[j], s1, ks1, qsw[j / 2]);
    } else {
      s0 = mfma_fp4_sel<2>(k0, qa[j], s0, ks0, qsw[j / 2]);
      s1 = mfma_fp4_sel<2>(k1, qa[j], s1, ks1, qsw[j / 2]);
    }
  }
}

template <int D>
constexpr int prefill_min_blocks() { return D >= 256 ? 1 : 2; }  // also used by decode

template <int D, bool kCausal>
__global__ __launch_bounds__(256, prefill_min_blocks<D>()) void attn_prefill_kernel(
    AttnArgs a, int ones_scale) {
  using T = PrefillTile<D>;
  constexpr int DB = T::DB, DS = T::DS;
  constexpr int NJ = D / 64;  // QK MFMAs per 32-key tile
  constexpr int NC = D / 32;  // P V channel tiles
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[2 * T::LDS_K];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[2 * T::LDS_V];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, n = lane & 31;

  // Work item.  Linear order: kv head fastest (so the query heads of one GQA
  // group, which read the same K / V, land on the same XCD when B*Hkv is a
  // multiple of 8), then the query head within the group, then query tiles
  // from the last (most keys under a causal mask) to the first.
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
  const int nblk_valid = (L + 31) / 32;
  const int nblk_cap = (a.cap + 31) / 32;

  // Q operand (B of S^T = K Q^T): query q, K blocks of 32 along d; its scale
  // bytes packed so that MFMA j reads byte 2*(j%2) of word j/2.
  uint4 qa[NJ];
  int qsw[(NJ + 1) / 2];
  if (q < a.Sq) {
    const uint8_t* qc = a.q_codes + (bhq * a.Sq + q) * DB;
    const uint8_t* qsc = a.q_scales + (bhq * a.Sq + q) * DS;
#pragma unroll
    for (int j = 0; j < NJ; j++) qa[j] = *reinterpret_cast<const uint4*>(qc + 32 * j + 16 * h);
#pragma unroll
    for (int j = 0; j < NJ; j += 2) qsw[j / 2] = k_scale_word<DS>(qsc, j, h);
  } else {
#pragma unroll
    for (int j = 0; j < NJ; j++) qa[j] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < NJ; j += 2) qsw[j / 2] = 0;
  }

  // Key ranges: the workgroup stages every tile any of its rows can see; a
  // wave computes only tiles its own rows can see; tiles below wave_full are
  // visible to every row of the wave (no mask needed).
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
  const int row_lim = kCausal ? min(L, q + L - a.Sq + 1) : L;  // keys < row_lim visible

  const uint32_t one_bits = n == 0 ? 0x22222222u : 0u;  // E2M1 1.0 in every nibble of row 0
  const uint4 ones = make_uint4(one_bits, one_bits, one_bits, one_bits);
  const float c = a.sm_log2;

  float m_run = -INFINITY;
  uint4 pk = make_uint4(0, 0, 0, 0);
  v16f acc[NC];
#pragma unroll
  for (int cc = 0; cc < NC; cc++) acc[cc] = v16f{};
  v16f accl = v16f{};

  // prologue: K tiles 0 and 1, V tile 0; scores of tile 0
  KRegs<D> kpre;
  VRegs<D> vpre;
  if (n_tiles > 0) {
    load_k<D>(a, bkv, 0, L, tid, kpre);
    load_v<D>(a, bkv, 0, nblk_valid, nblk_cap, tid, vpre);
    store_k<D>(lds_k, tid, kpre);
    store_v<D>(lds_v, tid, vpre);
    if (n_tiles > 1) {
      load_k<D>(a, bkv, kBN, L, tid, kpre);
      store_k<D>(lds_k + T::LDS_K, tid, kpre);
    }
  }
  // Drain every outstanding load on all paths into the loop.  Without it the
  // compiler must assume the Q operand loads may still be in flight at the
  // loop header (the prologue's loads are conditional) and makes the Q K^T
  // MFMAs of each step wait on the vector-memory counter, i.e. on the
  // prefetch loads issued just before them.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // One pipeline step: scores of tile kt are in (c0, c1); the next tile's go
  // to (n0r, n1r).  The loop below alternates the two register sets, so no
  // copies are needed; registers of a tile a wave does not compute are never
  // read (the softmax of that tile is skipped as well).  P is the parity of
  // kt, a compile-time constant, so every LDS address is a per-lane base plus
  // an immediate offset.
  auto step = [&](auto parity, int kt, v16f& c0, v16f& c1, v16f& n0r, v16f& n1r) {
    constexpr int P = decltype(parity)::value;
    const int n0 = kt * kBN;
    const bool more_k = kt + 2 < n_tiles, more_v = kt + 1 < n_tiles;
    if (more_k) load_k<D>(a, bkv, n0 + 2 * kBN, L, tid, kpre);
    if (more_v) load_v<D>(a, bkv, n0 + kBN, nblk_valid, nblk_cap, tid, vpre);

    // scores of the next tile go to the matrix core first
    if (more_v && n0 + kBN < wave_end)
      qk_step<D>(lds_k + (1 - P) * T::LDS_K, qa, qsw, n, h, n0r, n1r);
    __builtin_amdgcn_sched_barrier(0);

    if (n0 < wave_end) {  // uniform per wave
      if (n0 + kBN > wave_full) mask_scores(c0, c1, n0 + 32 * h, row_lim);
      const SoftmaxStep st = softmax_step(c0, c1, m_run, c, a.tau, pk);
      // rescale only when some row's max moved (multiplying by 1 is exact)
      if (__any(st.alpha != 1.0f)) {
#pragma unroll
        for (int cc = 0; cc < NC; cc++) acc[cc] *= st.alpha;
        accl[0] *= st.alpha;
      }

      // ---- [acc | l] += P_hat [V | 1]
      const uint8_t* vbuf = lds_v + P * T::LDS_V;
#pragma unroll
      for (int cc = 0; cc < NC; cc++) {
        const int ch = 32 * cc + n;
        const uint4 va = *reinterpret_cast<const uint4*>(vbuf + (h * D + ch) * 16);
        const int vs = vbuf[T::VC * 16 + h * D + ch];
        acc[cc] = mfma_fp4_32x32x64(va, st.p_codes, acc[cc], vs, st.p_scale);
      }
      accl = mfma_fp4_32x32x64(ones, st.p_codes, accl, ones_scale, st.p_scale);
    }
    if (more_k) store_k<D>(lds_k + P * T::LDS_K, tid, kpre);
    if (more_v) store_v<D>(lds_v + (1 - P) * T::LDS_V, tid, vpre);
    // Every load of this step has been consumed by now; saying so on all
    // paths keeps the compiler from assuming a load skipped by a branch is
    // still in flight, which would make the next step's prefetch loads wait
    // for one another.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  v16f sa0, sa1, sb0, sb1;
  if (0 < wave_end) qk_step<D>(lds_k, qa, qsw, n, h, sa0, sa1);
  for (int kt = 0; kt < n_tiles; kt += 2) {
    step(std::integral_constant<int, 0>{}, kt, sa0, sa1, sb0, sb1);
    if (kt + 1 < n_tiles) step(std::integral_constant<int, 1>{}, kt + 1, sb0, sb1, sa0, sa1);
  }

  // ---- epilogue: O = acc / l, LSE = m ln2 + ln l
  const float lsum = __shfl(accl[0], n);
  if (q < a.Sq) {
    const int64_t row = bhq * a.Sq + q;
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
    write_out<NC>(a, row, h, acc, inv);
    if (a.lse && h == 0) a.lse[row] = lsum > 0.0f ? m_run * kLn2 + logf(lsum) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Decode (Sq == 1), split-K: one wave = one chunk of `a.chunk` keys of one
// (batch, kv head) against the G query heads of that group (the MFMA's 32
// query columns, G used).  Each wave starts from a fresh state and writes its
// partial (m, l, acc[d]) to the workspace; the merge kernel combines them.
// K / V operands are loaded straight from global memory (each byte is read
// once), one 64-key tile ahead of the one being computed, so a wave always
// has a tile of HBM reads in flight behind its MFMA / softmax work.  Rows
// and blocks past the valid keys are clamped to the last valid one (finite
// data, masked scores, zero P).
// ---------------------------------------------------------------------------
template <int D>
struct DecTile {
  uint4 k0[D / 64], k1[D / 64];
  uint32_t ks0[(D / 64 + 1) / 2], ks1[(D / 64 + 1) / 2];  // raw scale words (shifted at use)
  uint4 va[D / 32];
  int vs[D / 32];
};

// Raw 32-bit word holding the scale byte of K block 2j + h of a row.
template <int DS>
__device__ __forceinline__ uint32_t k_scale_raw(const uint8_t* p, int j) {
  if constexpr (DS == 2) {
    return *reinterpret_cast<const uint16_t*>(p);
  } else {
    return reinterpret_cast<const uint32_t*>(p)[j >> 1];
  }
}

// Loads of the 64-key tile at n0.  Keys past last_key (and V blocks past
// last_blk) are clamped to it, so the load count is the same for every tile,
// including the prefetch past the end of the chunk (a re-read of rows just
// loaded).  A fixed count lets each step wait for exactly the tile it uses.
template <int D>
__device__ __forceinline__ void dec_load(const AttnArgs& a, int64_t bkv, int n0, int last_key,
                                         int last_blk, int nblk_cap, int r0, int r1, int n,
                                         int h, DecTile<D>& t) {
  constexpr int DB = D / 2, DS = D / 32, NJ = D / 64, NC = D / 32;
  const int64_t k0row = bkv * a.cap + min(n0 + r0, last_key);
  const int64_t k1row = bkv * a.cap + min(n0 + r1, last_key);
  const uint8_t* kc0 = a.k_codes + k0row * DB + 16 * h;
  const uint8_t* kc1 = a.k_codes + k1row * DB + 16 * h;
#pragma unroll
  for (int j = 0; j < NJ; j++) {
    t.k0[j] = *reinterpret_cast<const uint4*>(kc0 + 32 * j);
    t.k1[j] = *reinterpret_cast<const uint4*>(kc1 + 32 * j);
  }
#pragma unroll
  for (int j = 0; j < NJ; j += 2) {
    t.ks0[j / 2] = k_scale_raw<DS>(a.k_scales + k0row * DS, j);
    t.ks1[j / 2] = k_scale_raw<DS>(a.k_scales + k1row * DS, j);
  }
  const int64_t vb = bkv * nblk_cap + min(n0 / 32 + h, last_blk);
#pragma unroll
  for (int cc = 0; cc < NC; cc++) {
    t.va[cc] = *reinterpret_cast<const uint4*>(a.v_codes + (vb * D + 32 * cc + n) * 16);
    t.vs[cc] = a.v_scales[vb * D + 32 * cc + n];
  }
}

template <int D>
__global__ __launch_bounds__(256, prefill_min_blocks<D>()) void attn_decode_split_kernel(AttnArgs a,
                                                                                  int ones_scale) {
  constexpr int DB = D / 2, DS = D / 32, NJ = D / 64, NC = D / 32;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, n = lane & 31;
  const int G = a.Hq / a.Hkv;
  const int bkv_i = blockIdx.y;
  const int b = bkv_i / a.Hkv, g = bkv_i % a.Hkv;
  const int64_t bkv = (int64_t)b * a.Hkv + g;
  int L = a.Sk;
  if (a.kv_lens) L = min(max(a.kv_lens[b], 0), a.Sk);
  const int chunk_idx = blockIdx.x * kWaves + wave;
  const int s0 = chunk_idx * a.chunk;
  if (s0 >= L) return;  // uniform per wave; no barriers below
  const int s1 = min(L, s0 + a.chunk);
  const int nblk_cap = (a.cap + 31) / 32;

  // Q operand: column n is query head g*G + n (zero for n >= G).
  uint4 qa[NJ];
  int qsw[(NJ + 1) / 2];
  if (n < G) {
    const int64_t row = ((int64_t)b * a.Hq + g * G + n);  // Sq == 1
    const uint8_t* qc = a.q_codes + row * DB;
    const uint8_t* qsc = a.q_scales + row * DS;
#pragma unroll
    for (int j = 0; j < NJ; j++) qa[j] = *reinterpret_cast<const uint4*>(qc + 32 * j + 16 * h);
#pragma unroll
    for (int j = 0; j < NJ; j += 2) qsw[j / 2] = k_scale_word<DS>(qsc, j, h);
  } else {
#pragma unroll
    for (int j = 0; j < NJ; j++) qa[j] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < NJ; j += 2) qsw[j / 2] = 0;
  }
  const uint32_t one_bits = n == 0 ? 0x22222222u : 0u;
  const uint4 ones = make_uint4(one_bits, one_bits, one_bits, one_bits);
  const float c = a.sm_log2;
  float m_run = -INFINITY;
  uint4 pk = make_uint4(0, 0, 0, 0);
  v16f acc[NC];
#pragma unroll
  for (int cc = 0; cc < NC; cc++) acc[cc] = v16f{};
  v16f accl = v16f{};
  const int r0 = perm_row(0, n), r1 = perm_row(1, n);
  const int last_key = s1 - 1, last_blk = (s1 - 1) / 32;

  // one 64-key step on the tile in `cur`, with the next tile's loads issued
  // into `nxt` first
  auto step = [&](int n0, const DecTile<D>& cur, DecTile<D>& nxt) {
    dec_load<D>(a, bkv, n0 + kBN, last_key, last_blk, nblk_cap, r0, r1, n, h, nxt);
    v16f t0 = v16f{}, t1 = v16f{};
#pragma unroll
    for (int j = 0; j < NJ; j++) {
      const int ks0 = (int)(cur.ks0[j / 2] >> (8 * h)), ks1 = (int)(cur.ks1[j / 2] >> (8 * h));
      if (j % 2 == 0) {
        t0 = mfma_fp4_sel<0>(cur.k0[j], qa[j], t0, ks0, qsw[j / 2]);
        t1 = mfma_fp4_sel<0>(cur.k1[j], qa[j], t1, ks1, qsw[j / 2]);
      } else {
        t0 = mfma_fp4_sel<2>(cur.k0[j], qa[j], t0, ks0, qsw[j / 2]);
        t1 = mfma_fp4_sel<2>(cur.k1[j], qa[j], t1, ks1, qsw[j / 2]);
      }
    }
    if (n0 + kBN > s1) mask_scores(t0, t1, n0 + 32 * h, s1);
    const SoftmaxStep st = softmax_step(t0, t1, m_run, c, a.tau, pk);
    if (__any(st.alpha != 1.0f)) {
#pragma unroll
      for (int cc = 0; cc < NC; cc++) acc[cc] *= st.alpha;
      accl[0] *= st.alpha;
    }
#pragma unroll
    for (int cc = 0; cc < NC; cc++)
      acc[cc] = mfma_fp4_32x32x64(cur.va[cc], st.p_codes, acc[cc], cur.vs[cc], st.p_scale);
    accl = mfma_fp4_32x32x64(ones, st.p_codes, accl, ones_scale, st.p_scale);
  };

  DecTile<D> ta, tb;
  dec_load<D>(a, bkv, s0, last_key, last_blk, nblk_cap, r0, r1, n, h, ta);
  for (int n0 = s0; n0 < s1; n0 += 2 * kBN) {
    step(n0, ta, tb);
    if (n0 + kBN < s1) step(n0 + kBN, tb, ta);
  }

  // partial row: [m, l, acc[0..D)] for (b, query head, chunk)
  const float lsum = __shfl(accl[0], n);
  if (n < G) {
    float* part = a.partials + (((int64_t)b * a.Hq + g * G + n) * a.n_chunks + chunk_idx) * (D + 2);
    if (h == 0) {
      part[0] = m_run;
      part[1] = lsum;
    }
#pragma unroll
    for (int cc = 0; cc < NC; cc++)
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        const int ch = 32 * cc + 8 * g4 + 4 * h;
#pragma unroll
        for (int i = 0; i < 4; i++) part[2 + ch + i] = acc[cc][4 * g4 + i];
      }
  }
}

// Log-sum-exp merge of the chunk partials: one wave per (batch, query head).
// Lane i owns chunk i (and i + 64, ...) for the max and the normaliser (wave
// reductions); the accumulators are combined channel-parallel, eight chunks
// per round so that eight partial rows are in flight at once.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

template <int D>
__global__ __launch_bounds__(256) void attn_decode_merge_kernel(AttnArgs a) {
  constexpr int CPL = (D + 63) / 64;  // channels per lane
  constexpr int U = 8;                // chunks per round
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);  // b * Hq + hq
  if (row >= (int64_t)a.B * a.Hq) return;
  const int b = (int)(row / a.Hq);
  int L = a.Sk;
  if (a.kv_lens) L = min(max(a.kv_lens[b], 0), a.Sk);
  const int nc = (L + a.chunk - 1) / a.chunk;
  const float* part = a.partials + row * a.n_chunks * (D + 2);
  float M = -INFINITY;
  for (int i = lane; i < nc; i += 64) M = fmaxf(M, part[(int64_t)i * (D + 2)]);
  M = wave_max(M);
  float lpart = 0.0f;
  for (int i = lane; i < nc; i += 64) {
    const float* pr = part + (int64_t)i * (D + 2);
    lpart += fast_exp2(pr[0] - M) * pr[1];
  }
  const float lsum = M == -INFINITY ? 0.0f : wave_sum(lpart);
  float o[CPL];
#pragma unroll
  for (int j = 0; j < CPL; j++) o[j] = 0.0f;
  for (int i0 = 0; i0 < nc; i0 += U) {
    float w[U], x[U][CPL];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int i = min(i0 + u, nc - 1);
      const float* pr = part + (int64_t)i * (D + 2);
      w[u] = (i0 + u < nc && M != -INFINITY) ? fast_exp2(pr[0] - M) : 0.0f;
#pragma unroll
      for (int j = 0; j < CPL; j++) {
        const int ch = lane + 64 * j;
        x[u][j] = ch < D ? pr[2 + ch] : 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; u++)
#pragma unroll
      for (int j = 0; j < CPL; j++) o[j] += w[u] * x[u][j];
  }
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
#pragma unroll
  for (int j = 0; j < CPL; j++) {
    const int ch = lane + 64 * j;
    if (ch < D) {
      const float v = o[j] * inv;
      static_cast<uint16_t*>(a.out)[row * D + ch] =
          (uint16_t)(a.out_fp16 ? float_to_half_bits(v) : float_to_bf16_bits(v));
    }
  }
  if (a.lse && lane == 0) a.lse[row] = lsum > 0.0f ? M * kLn2 + logf(lsum) : -INFINITY;
}

// The E8M0 byte for 2^0, passed as a kernel argument: the scaled MFMA must
// see its scale operands as integer registers, not as a folded constant.
constexpr int kScaleOne = 127;

template <int D>
hipError_t launch_prefill_d(const AttnArgs& a, hipStream_t stream) {
  const int n_qt = (a.Sq + kBR - 1) / kBR;
  const int64_t grid = (int64_t)n_qt * a.B * a.Hq;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (a.causal)
    hipLaunchKernelGGL((attn_prefill_kernel<D, true>), dim3((unsigned)grid), dim3(256), 0, stream,
                       a, kScaleOne);
  else
    hipLaunchKernelGGL((attn_prefill_kernel<D, false>), dim3((unsigned)grid), dim3(256), 0, stream,
                       a, kScaleOne);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const AttnArgs& a, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  if (a.Hq / a.Hkv > 32) return hipErrorNotSupported;  // one MFMA column per query head
  const int wg_x = (a.n_chunks + kWaves - 1) / kWaves;
  if (wg_x > 0) {
    hipLaunchKernelGGL(attn_decode_split_kernel<D>, dim3(wg_x, a.B * a.Hkv), dim3(256), 0, stream,
                       a, kScaleOne);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t rows = (int64_t)a.B * a.Hq;
  hipLaunchKernelGGL(attn_decode_merge_kernel<D>, dim3((unsigned)((rows + kWaves - 1) / kWaves)),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int attn_block_n(int) { return kBN; }
int attn_default_chunk(int) { return kDecodeChunk; }

hipError_t launch_attn_prefill_mxfp4(const AttnArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 64: return launch_prefill_d<64>(a, stream);
    case 128: return launch_prefill_d<128>(a, stream);
    case 256: return launch_prefill_d<256>(a, stream);
  }
  return hipErrorNotSupported;
}

hipError_t launch_attn_decode_mxfp4(const AttnArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 64: return launch_decode_d<64>(a, stream);
    case 128: return launch_decode_d<128>(a, stream);
    case 256: return launch_decode_d<256>(a, stream);
  }
  return hipErrorNotSupported;
}

}  // namespace hifa4
