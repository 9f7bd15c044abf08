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
#include <utility>

#include "device_common.hpp"
#include "launch.hpp"
#include "lds_dma.hpp"

// Products and sums are rounded separately unless fmaf is spelled out: the
// softmax relies on fl(S * c) being the same value in the max and in the
// block-scale exponent.
#pragma clang fp contract(off)

namespace hifa4 {

namespace {

constexpr int kBN = 64;            // keys per online-softmax step (the P frame tile)
static_assert(kBN == 64, "decode_piece_tiles counts 64-key tiles");
constexpr int kWaves = 4;          // waves per workgroup
constexpr int kBR = 32 * kWaves;   // queries per prefill workgroup
constexpr float kLn2 = 0.6931471805599453f;

// Row of the 64-key step that A-operand row m of 32-key tile t loads.
__device__ __forceinline__ int perm_row(int t, int m) {
  return 32 * ((m >> 2) & 1) + 16 * t + 4 * (m >> 3) + (m & 3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Result of an online-softmax step on the 32 scores a lane holds for its
// query: the packed P operand, its E8M0 byte and the accumulators' rescale
// factor.
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

// Non-reordered normaliser: the sum of the row's fp32 P over the 64 keys of a
// step (the lane's 32 in the two accumulators after the exponentials, plus the
// partner lane's 32), as a tree of adds.
__device__ __forceinline__ float row_sum_p(const v16f& p0, const v16f& p1) {
  float t[16];
#pragma unroll
  for (int r = 0; r < 16; r++) t[r] = p0[r] + p1[r];
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
    for (int r = 0; r < w; r++) t[r] = t[r] + t[r + w];
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(t[0]), __float_as_uint(t[0]),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Softmax on the lane's 32 scores held in the two QK accumulators (tile t,
// register r <-> key 32h + 16t + r), in place: the scores are replaced by P
// before packing, so no copies of the accumulators are made.  Masked scores
// are -inf on entry.
//
// The two halves of a softmax step, so that the Q K^T MFMAs of the next tile
// can be issued between them: softmax_max() finds the new running max and
// the rescale factor, softmax_exp() turns the scores into P and packs it.
struct SoftmaxMax {
  float m_use;  // the frame P is taken in (0 while the row has seen no key)
  float bmc;    // fl(block max of S * c)
  float alpha;  // rescale factor of the accumulators
  bool moved;   // kLazyAlpha: some row of the wave moved its frame (uniform)
};

// kLazyAlpha: alpha = 1 without its exponential unless some row of the wave
// moved its frame (a uniform branch; with the lazy threshold most steps move
// none).  Where it is computed it is the same exp2(m_run - m_use); a row that
// has seen no key keeps alpha = 1 instead of 0, which scales its still-zero
// accumulators the same way.
template <bool kLazyAlpha = false>
__device__ __forceinline__ SoftmaxMax softmax_max(const v16f& s0, const v16f& s1, float& m_run,
                                                  float c, float tau) {
  // max3 tree over the 32 scores (32 -> 11 -> 4 -> 1): depth 4 instead of
  // two chains of 8
  float t[32];
#pragma unroll
  for (int r = 0; r < 16; r++) {
    t[r] = s0[r];
    t[16 + r] = s1[r];
  }
  float u[11];
#pragma unroll
  for (int i = 0; i < 10; i++) u[i] = fmax_(fmax_(t[3 * i], t[3 * i + 1]), t[3 * i + 2]);
  u[10] = fmax_(t[30], t[31]);
  const float v0 = fmax_(fmax_(u[0], u[1]), u[2]), v1 = fmax_(fmax_(u[3], u[4]), u[5]);
  const float v2 = fmax_(fmax_(u[6], u[7]), u[8]), v3 = fmax_(u[9], u[10]);
  const float bm = fmax_(fmax_(v0, v1), fmax_(v2, v3));
  SoftmaxMax x;
  x.bmc = bm * c;  // contraction is off in this file: a rounded product
  const float rmc = max_with_half_swap(x.bmc);
  const float m_new = rmc > m_run + tau ? rmc : m_run;
  x.m_use = m_new == -INFINITY ? 0.0f : m_new;
  if constexpr (kLazyAlpha) {
    x.moved = __any(m_new != m_run);
    x.alpha = 1.0f;
    if (x.moved) x.alpha = fast_exp2(m_run - x.m_use);
  } else {
    x.moved = true;
    x.alpha = fast_exp2(m_run - x.m_use);
  }
  m_run = m_new;
  return x;
}

// `pk` is the previous step's packed P: every byte of it is overwritten, it
// only gives the partial-write converts a register to start from.
__device__ __forceinline__ SoftmaxStep softmax_exp(v16f& s0, v16f& s1, const SoftmaxMax& x,
                                                   float c, uint32_t p_bias, uint4& pk) {
#pragma unroll
  for (int r = 0; r < 16; r++) {
    s0[r] = fast_exp2(__builtin_fmaf(s0[r], c, -x.m_use));
    s1[r] = fast_exp2(__builtin_fmaf(s1[r], c, -x.m_use));
  }
  const float pmax = fast_exp2(x.bmc - x.m_use);
  const uint32_t sb = e8m0_from_amax(pmax, p_bias);
  SoftmaxStep st;
  st.alpha = x.alpha;
  st.p_scale = (int)sb;
  const float scale = e8m0_to_float(sb);
  uint32_t w[4] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const v16f& src = q < 2 ? s0 : s1;
    const int o = 8 * (q & 1);
    uint32_t v = w[q];
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, src[o + 0], src[o + 1], scale, 0);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, src[o + 2], src[o + 3], scale, 1);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, src[o + 4], src[o + 5], scale, 2);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, src[o + 6], src[o + 7], scale, 3);
    w[q] = v;
  }
  st.p_codes = make_uint4(w[0], w[1], w[2], w[3]);
  pk = st.p_codes;
  return st;
}

// Whole step (decode): max phase then exp phase.
__device__ __forceinline__ SoftmaxStep softmax_step(v16f& s0, v16f& s1, float& m_run, float c,
                                                    float tau, uint32_t p_bias, uint4& pk) {
  const SoftmaxMax x = softmax_max(s0, s1, m_run, c, tau);
  return softmax_exp(s0, s1, x, c, p_bias, pk);
}

// Mask keys >= lim (key of element (t, r) is kb + 16t + r) with -inf.  The
// keep / drop decision is the sign of (lim - 1 - key), spread over the word
// by an arithmetic shift and merged with a bitfield select: no compare
// masks, which would each take a pair of scalar registers.
__device__ __forceinline__ float keep_or_neg_inf(float x, int last_minus_key) {
  const uint32_t drop = (uint32_t)(last_minus_key >> 31);  // all ones if key > last
  return __uint_as_float((__float_as_uint(x) & ~drop) | (0xFF800000u & drop));
}

__device__ __forceinline__ void mask_scores(v16f& s0, v16f& s1, int kb, int lim) {
  const int rem = lim - 1 - kb;  // element r is kept iff r <= rem
#pragma unroll
  for (int r = 0; r < 16; r++) {
    s0[r] = keep_or_neg_inf(s0[r], rem - r);
    s1[r] = keep_or_neg_inf(s1[r], rem - 16 - r);
  }
}

// Output tile of a wave (rows row0 .. row0 + nrows - 1, nrows <= 32) through
// LDS.  Each half-wave holds 4 of every 8 consecutive channels of its query's
// row; one lane swap per dword (lane n with lane n + 32) gives every lane 8
// consecutive channels of one group, written to the staging rows as 16 bytes.
// The tile then goes to memory as whole rows: lane l stores 16 bytes of row
// l / (D / 8) of each group of 512 / D rows, so a store instruction writes
// 1 KB in full 128-byte lines instead of 32 bytes in each of 32 rows
// (measured 2-3.6 % faster over the whole launch on the Gemma2-, Llama- and
// Qwen3-shaped prefill layers, same bits).
template <int NC, bool kHalf>
__device__ __forceinline__ void write_out(const AttnArgs& a, int64_t row0, int nrows, int n,
                                          int h, int lane, const v16f (&acc)[NC], float inv,
                                          uint8_t* stage) {
  constexpr int D = NC * 32;
  constexpr int STRIDE = 2 * D + 16;
  // two channels to one packed word with the hardware's round-to-nearest-even
  // converts (gfx950 packs two fp32 into bf16 / fp16 in one instruction)
  auto cvt2 = [&](float x, float y) -> uint32_t {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const f2 v = {x, y};
    if constexpr (kHalf)
      return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));
    else
      return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
  };
#pragma unroll
  for (int c = 0; c < NC; c++) {
#pragma unroll
    for (int gp = 0; gp < 2; gp++) {
      // groups ga (kept by the lower half-wave) and gb (upper): lane (n, h)
      // holds channels 8 g + 4 h .. + 3 of both
      const int ga = 2 * gp, gb = 2 * gp + 1;
      const uint32_t a0 = cvt2(acc[c][4 * ga] * inv, acc[c][4 * ga + 1] * inv);
      const uint32_t a1 = cvt2(acc[c][4 * ga + 2] * inv, acc[c][4 * ga + 3] * inv);
      const uint32_t b0 = cvt2(acc[c][4 * gb] * inv, acc[c][4 * gb + 1] * inv);
      const uint32_t b1 = cvt2(acc[c][4 * gb + 2] * inv, acc[c][4 * gb + 3] * inv);
      // the upper half's group-ga words go down, the lower half's group-gb words up
      const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
      const int ch = 32 * c + 8 * (h ? gb : ga);
      *reinterpret_cast<uint4*>(stage + n * STRIDE + 2 * ch) = make_uint4(s0[0], s1[0], s0[1], s1[1]);
    }
  }
  constexpr int LPR = D / 8;    // lanes per row (16 bytes each)
  constexpr int RPI = 64 / LPR; // rows per store instruction
  const int rr = lane / LPR, cb = (lane % LPR) * 16;
  uint8_t* out = static_cast<uint8_t*>(a.out);
#pragma unroll
  for (int k = 0; k < 32 / RPI; k++) {
    const int r = k * RPI + rr;
    const uint4 v = *reinterpret_cast<const uint4*>(stage + r * STRIDE + cb);
    if (r < nrows) *reinterpret_cast<uint4*>(out + (row0 + r) * (2 * D) + cb) = v;
  }
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

// ---------------------------------------------------------------------------
// Prefill: one workgroup = 128 queries of one (batch, query head); 4 waves of
// 32 queries share 64-key K / V tiles staged in LDS.
//
// Software pipeline.  Step kt of a wave issues the Q K^T MFMAs of tile kt+1
// first, then runs the softmax of tile kt (whose scores came out of the
// previous step) and its P V MFMAs: the matrix core computes the next scores
// while the vector ALU does the exponentials and FP4 conversions.
//
// Staging.  K and V tiles go from memory straight into LDS (buffer loads
// with the LDS destination: no registers, no LDS store instructions) through
// rings of four buffers.  Step kt reads K tile kt+1 and V tile kt and issues
// the loads of K tile kt+3 and V tile kt+2 into the buffers the previous
// step finished with; before its closing barrier it waits only for the loads
// issued one step earlier (K tile kt+2, V tile kt+1), so every load has two
// steps of compute to arrive.  Each wave loads a quarter of every tile and
// issues the same number of loads each step (past the last tile with an
// empty descriptor range), so a fixed vmcnt(N) wait is exact.
//
// The loads are written in inline asm: the compiler then neither makes LDS
// reads of other buffers wait for them nor drains them at the barrier, and
// the explicit vector-memory waits below are the synchronisation.  They have
// no register results.
//
// K layout in LDS: dense rows of d/2 bytes in the order the MFMA A operand
// reads them (row R = 32t + n holds key perm_row(t, n)), the 16-byte chunks
// of row R XOR-swizzled by k_swz(R) so that the 16-byte reads of
// neighbouring lanes fall in distinct banks; the scale bytes follow in the
// same row order, max(d/32, 4) bytes per row.  V keeps its global layout
// (key-blocked, channel-major).
// The permutation and the swizzle are applied on the global side: lane i of
// a load writes LDS bytes 16i .. 16i+15 and fetches whatever belongs there.
// ---------------------------------------------------------------------------
template <int D>
struct PrefillTile {
  static constexpr int DB = D / 2;    // code bytes per K row
  static constexpr int DS = D / 32;   // scale bytes per K row
  static constexpr int NCH = DB / 16; // 16-byte chunks per K row
  static constexpr int RPB_SHIFT = D == 64 ? 2 : (D == 128 ? 1 : 0);  // log2(K rows per 128 B)
  static constexpr int KSS = DS < 4 ? 4 : DS;        // LDS slot of one row's K scales
  static constexpr int KS_OFF = kBN * DB;            // K scales within a K stage
  static constexpr int K_BYTES = KS_OFF + kBN * KSS; // one K stage
  static constexpr int VS_OFF = 2 * D * 16;          // V scales within a V stage
  static constexpr int V_BYTES = VS_OFF + 2 * D;     // one V stage
  // Per wave and tile: 16-byte K / V code chunks, K scale lanes (one row per
  // lane, two lanes per row when a row has 8 scale bytes) and 4-byte V scale
  // words.
  static constexpr int KC_W = DB;
  static constexpr int VC_W = D / 2;
  static constexpr int KS_W = DS == 8 ? 32 : 16;
  static constexpr int VS_W = D / 8;
  static constexpr int KC_I = (KC_W + 63) / 64;  // load instructions for them
  static constexpr int VC_I = (VC_W + 63) / 64;
  static constexpr int N_LOADS = KC_I + VC_I + 2;  // per wave and step
  static constexpr int STAGES = 4;                 // ring depth (K and V)
  // Output staging after the last step: a wave's 32 x D tile, rows padded by
  // 16 bytes (row r starts 4 banks after row r - 1, so the 16-byte writes of
  // 16 consecutive rows fall in distinct banks).  At d = 64 each wave has a
  // region of its own, written and read by that wave alone; at d = 128 (three
  // workgroups per CU) and d = 256 there is no room beside the rings, so
  // after a workgroup barrier waves 0, 1 use the K ring and waves 2, 3 the V
  // ring.
  static constexpr int OUT_STRIDE = 2 * D + 16;
  static constexpr int OUT_TILE = 32 * OUT_STRIDE;
  static constexpr bool OUT_OWN = D <= 64;
  static constexpr int K_RING = OUT_OWN || STAGES * K_BYTES >= 2 * OUT_TILE ? STAGES * K_BYTES : 2 * OUT_TILE;
  static constexpr int V_RING = OUT_OWN || STAGES * V_BYTES >= 2 * OUT_TILE ? STAGES * V_BYTES : 2 * OUT_TILE;
  static_assert(N_LOADS < 16, "vmcnt encoding below assumes fewer than 16");
};

template <int D>
__device__ __forceinline__ int k_swz(int R) {
  using T = PrefillTile<D>;
  return ((R >> T::RPB_SHIFT) ^ (R >> 3)) & (T::NCH - 1);
}

// Per-lane source offsets of a wave's share of a tile (loop invariant).
template <int D>
struct TileLanes {
  uint32_t kc[PrefillTile<D>::KC_I];
  uint32_t ks;
};

template <int D>
__device__ __forceinline__ TileLanes<D> tile_lanes(int w, int lane) {
  using T = PrefillTile<D>;
  TileLanes<D> tl;
#pragma unroll
  for (int i = 0; i < T::KC_I; i++) {
    const int b = w * T::KC_W + 64 * i + lane;  // chunk index in LDS order
    const int R = b / T::NCH, pos = b % T::NCH;
    const int key = perm_row(R >> 5, R & 31);
    tl.kc[i] = (uint32_t)(key * T::DB + ((pos ^ k_swz<D>(R)) * 16));
  }
  {
    // the wave's 16 rows 16w .. 16w + 15 (LDS order); 8-byte rows take two
    // lanes of 4 bytes each
    const int R = 16 * w + (T::DS == 8 ? lane >> 1 : lane);
    tl.ks = (uint32_t)(perm_row(R >> 5, R & 31) * T::DS + (T::DS == 8 ? 4 * (lane & 1) : 0));
  }
  return tl;
}

// Descriptors of one (batch, kv head): K codes / scales over the L valid
// keys, V codes / scales over the valid 32-key blocks.
struct HeadDescs {
  v4i kc, ks, vc, vs;
};

template <int D>
__device__ __forceinline__ HeadDescs head_descs(const AttnArgs& a, int64_t bkv, int L,
                                                int nblk_valid, int nblk_cap) {
  using T = PrefillTile<D>;
  HeadDescs hd;
  const int64_t row0 = bkv * a.cap;
  const int64_t blk0 = bkv * nblk_cap;
  hd.kc = buffer_desc(a.k_codes + row0 * T::DB, (uint32_t)L * T::DB);
  hd.ks = buffer_desc(a.k_scales + row0 * T::DS, (uint32_t)L * T::DS);
  hd.vc = buffer_desc(a.v_codes + blk0 * D * 16, (uint32_t)nblk_valid * D * 16);
  hd.vs = buffer_desc(a.v_scales + blk0 * D, (uint32_t)nblk_valid * D);
  return hd;
}

// A tile past the last one the workgroup needs reads nothing: its offset is
// put past every descriptor's range (the loads still count in vmcnt).
constexpr int kPastEnd = 0x7FFFFFF0;

// The wave's LDS destinations in stage 0 (other stages: + an immediate).
struct WaveDst {
  uint32_t kc, ks, vc, vs;
};

template <int D>
__device__ __forceinline__ WaveDst wave_dst(uint32_t k_base, uint32_t v_base, int w) {
  using T = PrefillTile<D>;
  WaveDst d;
  d.kc = k_base + w * T::KC_W * 16;
  d.ks = k_base + T::KS_OFF + 16 * w * T::KSS;
  d.vc = v_base + w * T::VC_W * 16;
  d.vs = v_base + T::VS_OFF + w * T::VS_W * 4;
  return d;
}

// Issue the wave's loads of K tile `tile` into K stage KST.
template <int D, int KST>
__device__ __forceinline__ void issue_k(const HeadDescs& hd, int tile, int n_tiles,
                                        const WaveDst& wd, int lane, const TileLanes<D>& tl) {
  using T = PrefillTile<D>;
  constexpr int SB = KST * T::K_BYTES;
  const bool live = tile < n_tiles;
  const int soc = live ? tile * kBN * T::DB : kPastEnd;
  const int sos = live ? tile * kBN * T::DS : kPastEnd;
  if (T::KC_W >= 64 || lane < T::KC_W) load_lds16<SB>(hd.kc, tl.kc[0], soc, wd.kc);
  if constexpr (T::KC_I > 1) load_lds16<SB + 1024>(hd.kc, tl.kc[1], soc, wd.kc);
  static_assert(T::KC_I <= 2, "at most two K code loads per wave");
  if (lane < T::KS_W) {
    if constexpr (T::DS == 2)
      load_lds2<SB>(hd.ks, tl.ks, sos, wd.ks);  // one row's 2 bytes, zero-extended into its slot
    else
      load_lds4<SB>(hd.ks, tl.ks, sos, wd.ks);
  }
}

template <int D, int VST>
__device__ __forceinline__ void issue_v(const HeadDescs& hd, int tile, int n_tiles,
                                        const WaveDst& wd, int lane, uint32_t vlane,
                                        uint32_t vslane) {
  using T = PrefillTile<D>;
  constexpr int SB = VST * T::V_BYTES;
  const bool live = tile < n_tiles;
  const int soc = live ? tile * 2 * D * 16 : kPastEnd;
  const int sos = live ? tile * 2 * D : kPastEnd;
  // vlane = (w * VC_W + lane) * 16 and vslane = (w * VS_W + lane) * 4: the
  // lane's code chunk and scale word in the wave's share (V keeps its layout)
  if (T::VC_W >= 64 || lane < T::VC_W) load_lds16<SB>(hd.vc, vlane, soc, wd.vc);
  if constexpr (T::VC_I > 1) load_lds16<SB + 1024>(hd.vc, vlane + 1024, soc, wd.vc);
  static_assert(T::VC_I <= 2, "at most two V code loads per wave");
  if (lane < T::VS_W) load_lds4<SB>(hd.vs, vslane, sos, wd.vs);
}

// K operands of the two 32-key tiles of a 64-key step, read from one K stage:
// koff[t][j] is the lane's byte offset of its 16-byte A chunk (row 32t + n,
// chunk 2j + h, swizzled).
template <int D>
struct KOps {
  uint4 k[2][D / 64];
  int ks[2][D / 64];
};

template <int D>
__device__ __forceinline__ void qk_load(const uint8_t* kbuf, const uint32_t (&koff)[2][D / 64],
                                        int n, int h, KOps<D>& o) {
  using T = PrefillTile<D>;
  const uint8_t* ks = kbuf + T::KS_OFF;
#pragma unroll
  for (int j = 0; j < D / 64; j++) {
    o.k[0][j] = *reinterpret_cast<const uint4*>(kbuf + koff[0][j]);
    o.k[1][j] = *reinterpret_cast<const uint4*>(kbuf + koff[1][j]);
    o.ks[0][j] = k_scale_word<T::DS>(ks + n * T::KSS, j, h);
    o.ks[1][j] = k_scale_word<T::DS>(ks + (32 + n) * T::KSS, j, h);
  }
}

// S^T = K Q^T for the two tiles.
template <int D>
__device__ __forceinline__ void qk_mfma(const KOps<D>& o, const uint4 (&qa)[D / 64],
                                        const int (&qsw)[(D / 64 + 1) / 2], v16f& s0, v16f& s1) {
  s0 = v16f{};
  s1 = v16f{};
#pragma unroll
  for (int j = 0; j < D / 64; j++) {
    if (j % 2 == 0) {
      s0 = mfma_fp4_sel<0>(o.k[0][j], qa[j], s0, o.ks[0][j], qsw[j / 2]);
      s1 = mfma_fp4_sel<0>(o.k[1][j], qa[j], s1, o.ks[1][j], qsw[j / 2]);
    } else {
      s0 = mfma_fp4_sel<2>(o.k[0][j], qa[j], s0, o.ks[0][j], qsw[j / 2]);
      s1 = mfma_fp4_sel<2>(o.k[1][j], qa[j], s1, o.ks[1][j], qsw[j / 2]);
    }
  }
}

// V operands of one tile for the P V MFMAs: lane (n, h) takes channel
// 32cc + n of key block h (16 code bytes) and its scale byte.
template <int D>
struct VOps {
  uint4 va[D / 32];
  int vs[D / 32];
};

template <int D>
__device__ __forceinline__ void v_load(const uint8_t* vbuf, int n, int h, VOps<D>& o) {
  using T = PrefillTile<D>;
#pragma unroll
  for (int cc = 0; cc < D / 32; cc++) {
    const int ch = 32 * cc + n;
    o.va[cc] = *reinterpret_cast<const uint4*>(vbuf + (h * D + ch) * 16);
    o.vs[cc] = vbuf[T::VS_OFF + h * D + ch];
  }
}

// Workgroups per compute unit (= waves per SIMD): three at d = 128 (154
// VGPRs, 34 KB of LDS each), two at d = 64 and d = 256 (the 32 x 256
// accumulator tile alone is 128 registers a lane).
template <int D>
constexpr int prefill_min_blocks() { return D == 128 ? 3 : 2; }

// d = 128 and d = 256 run the step in two phases, softmax then products,
// instead of interleaving the next tile's Q K^T with the current softmax in
// one wave: one S tile per wave instead of two, operands read from LDS just
// before their MFMA.  The waves sharing a SIMD take turns, one in its softmax
// while another keeps the matrix core busy.  At d = 256 this is what lets two
// waves fit a SIMD; at d = 128 it lets three fit (the interleaved step needs
// 221 registers): Llama-3.1-8B-shaped layer 163.0 -> 148.2 us, Qwen3-8B 71.4
// -> 70.4.  d = 64 keeps the interleaved step.
template <int D>
constexpr bool prefill_two_phase() { return D >= 128; }

// Smooth-QK (Q * s in fp32) and MXFP4 of the lane's blocks 2j + h (j < D/64)
// of query row `row`, from the bf16 / fp16 activations: the same arithmetic as
// the quantise kernel (products, exact block max, E8M0 exponent, packed
// convert), so the codes are bit-identical.  The scale byte of block 2j + h
// goes to byte h + 2 (j % 2) of word j / 2, the quantise kernel's row layout
// as the lane reads it.
//
// Every load (the lane's raw blocks and their smoothing factors) is issued
// before the first one is used, so the section costs one memory round trip;
// with the smoothing test inside the block loop, the compiler had split it
// into four dependent ones (3.0 -> ~2 us per work item on the Qwen3-8B shape).
// Used for d <= 128; d = 256 reads the rows as whole runs (below).
template <int D, bool kBf16, bool kSmooth, uint32_t kQBias>
__device__ __forceinline__ void quantise_q_lane(const AttnArgs& a, int64_t row, int hs, int h,
                                                uint4 (&qa)[D / 64],
                                                uint32_t (&qsw_raw)[(D / 64 + 1) / 2]) {
  constexpr int NJ = D / 64;
  const uint16_t* src = a.q_raw + row * D;
  const float* sm = a.smooth + (int64_t)hs * D;
  uint4 raw[NJ][4];
#pragma unroll
  for (int j = 0; j < NJ; j++) {
    const uint4* p = reinterpret_cast<const uint4*>(src + 32 * (2 * j + h));
#pragma unroll
    for (int i = 0; i < 4; i++) raw[j][i] = p[i];
  }
  float4 sf[kSmooth ? NJ : 1][8];
  if constexpr (kSmooth) {
#pragma unroll
    for (int j = 0; j < NJ; j++) {
      const float4* sp = reinterpret_cast<const float4*>(sm + 32 * (2 * j + h));
#pragma unroll
      for (int i = 0; i < 8; i++) sf[j][i] = sp[i];
    }
  }
#pragma unroll
  for (int j = 0; j < (NJ + 1) / 2; j++) qsw_raw[j] = 0;
#pragma unroll
  for (int j = 0; j < NJ; j++) {
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint32_t ws[4] = {raw[j][i].x, raw[j][i].y, raw[j][i].z, raw[j][i].w};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        v[8 * i + 2 * e] = elem<kBf16>(ws[e] & 0xFFFFu);
        v[8 * i + 2 * e + 1] = elem<kBf16>(ws[e] >> 16);
      }
    }
    if constexpr (kSmooth) {
#pragma unroll
      for (int i = 0; i < 8; i++) {
        v[4 * i] = v[4 * i] * sf[j][i].x;
        v[4 * i + 1] = v[4 * i + 1] * sf[j][i].y;
        v[4 * i + 2] = v[4 * i + 2] * sf[j][i].z;
        v[4 * i + 3] = v[4 * i + 3] * sf[j][i].w;
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(v[i]));
    const uint32_t sb = e8m0_from_amax(amax, kQBias);
    const float scale = e8m0_to_float(sb);
    uint32_t wd[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
      const float e8[8] = {v[8 * q4], v[8 * q4 + 1], v[8 * q4 + 2], v[8 * q4 + 3],
                           v[8 * q4 + 4], v[8 * q4 + 5], v[8 * q4 + 6], v[8 * q4 + 7]};
      wd[q4] = encode8(e8, scale);
    }
    qa[j] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    qsw_raw[j / 2] |= sb << (8 * (h + 2 * (j % 2)));
  }
}

// Q from the bf16 / fp16 activations, smoothed (Q * s in fp32) and quantised
// to MXFP4 in the prologue, with the quantise kernel's arithmetic and lane
// decomposition (products, exact block max, E8M0 exponent, packed convert), so
// the codes are bit-identical to quantise-then-attend.
//
// A wave's 32 rows are contiguous in memory and are read as whole 1 KB runs:
// lane l holds bytes 16 l .. 16 l + 15 of each run, 8 elements whose channel
// offset 8 l mod d is the same in every run, so the lane loads its 8 smoothing
// factors once.  Four consecutive lanes hold a 32-element block: two quad
// swaps give the block max, and each lane encodes its 8 elements to 4 code
// bytes.  Codes and scale bytes go to a per-wave staging area in LDS in the
// row layout of the quantised tensors, from which each lane reads its MFMA
// operand (row n, blocks 2j + h) and scale words as the codes path reads
// them from memory.  Used at d = 256, where the per-lane form (each lane
// loading its own blocks' 64-byte pieces and 32 smoothing factors per block)
// spent ~6 us per work item in this section; the whole launch on the
// Gemma2-9B-shaped layer: 212.5 -> 207.1 us.  At d = 128 the LDS round trip
// costs more than the coalescing saves (Llama-3.1-8B-shaped layer 164.8 ->
// 170.1 us), so d <= 128 keeps the per-lane form.
template <int D>
struct QRaw {
  static constexpr int NI = D / 16;           // 1 KB runs in a wave's 32 rows
  static constexpr int RPI = 512 / D;         // rows per run
  static constexpr int DBQ = D / 2;           // code bytes per row
  static constexpr int SSQ = D / 32 < 4 ? 4 : D / 32;  // staged scale bytes per row
  static constexpr int STAGE = 32 * (DBQ + SSQ);       // staging bytes per wave
  uint4 raw[NI];
  float4 f0, f1;
};

template <int D>
__device__ __forceinline__ void q_raw_load(const AttnArgs& a, int64_t row0, int nrows, int hs,
                                           int lane, QRaw<D>& qr) {
  using R = QRaw<D>;
  // the factors first: the first run's products then wait only for it
  if (a.smooth) {
    const float4* sp = reinterpret_cast<const float4*>(a.smooth + (int64_t)hs * D + (8 * lane) % D);
    qr.f0 = sp[0];
    qr.f1 = sp[1];
  }
  // rows past the sequence read its last row (no branch between the loads)
  // and are zeroed in q_raw_quantise
  const uint4* src = reinterpret_cast<const uint4*>(a.q_raw + row0 * D) + (8 * lane) % D / 8;
  const int rl = (8 * lane) / D;  // the lane's row within a run
#pragma unroll
  for (int k = 0; k < R::NI; k++) qr.raw[k] = src[min(k * R::RPI + rl, nrows - 1) * (D / 8)];
}

__device__ __forceinline__ float quad_max(float x) {
  // lanes 1,0,3,2 then 2,3,0,1 of each quad (DPP quad_perm)
  x = fmaxf(x, __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), 0xB1, 0xF, 0xF, false)));
  return fmaxf(x, __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), 0x4E, 0xF, 0xF, false)));
}

template <int D, bool kBf16, bool kSmooth, uint32_t kQBias>
__device__ __forceinline__ void q_raw_quantise(const QRaw<D>& qr, int nrows, int lane, int n, int h,
                                               uint8_t* stg, uint4 (&qa)[D / 64],
                                               uint32_t (&qsw_raw)[(D / 64 + 1) / 2]) {
  using R = QRaw<D>;
  constexpr int NJ = D / 64;
  uint8_t* sc = stg + 32 * R::DBQ;  // scale rows after the code rows
  const int j0 = (8 * lane) % D, rl = (8 * lane) / D;
  const float ff[8] = {qr.f0.x, qr.f0.y, qr.f0.z, qr.f0.w, qr.f1.x, qr.f1.y, qr.f1.z, qr.f1.w};
#pragma unroll
  for (int k = 0; k < R::NI; k++) {
    const int r = k * R::RPI + rl;
    const bool in = r < nrows;
    const uint32_t ws[4] = {in ? qr.raw[k].x : 0u, in ? qr.raw[k].y : 0u, in ? qr.raw[k].z : 0u,
                            in ? qr.raw[k].w : 0u};
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = elem<kBf16>(ws[i] & 0xFFFFu);
      v[2 * i + 1] = elem<kBf16>(ws[i] >> 16);
    }
    if constexpr (kSmooth) {
#pragma unroll
      for (int i = 0; i < 8; i++) v[i] = v[i] * ff[i];
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(v[i]));
    amax = quad_max(amax);
    const uint32_t sb = e8m0_from_amax(amax, kQBias);
    *reinterpret_cast<uint32_t*>(stg + r * R::DBQ + j0 / 2) = encode8(v, e8m0_to_float(sb));
    if ((lane & 3) == 0) sc[r * R::SSQ + j0 / 32] = (uint8_t)sb;
  }
#pragma unroll
  for (int j = 0; j < NJ; j++)
    qa[j] = *reinterpret_cast<const uint4*>(stg + n * R::DBQ + (2 * j + h) * 16);
#pragma unroll
  for (int j = 0; j < NJ; j += 2) {
    if constexpr (D == 64)  // two scale bytes per row, as the codes path reads them
      qsw_raw[j / 2] = *reinterpret_cast<const uint16_t*>(sc + n * R::SSQ);
    else
      qsw_raw[j / 2] = reinterpret_cast<const uint32_t*>(sc + n * R::SSQ)[j >> 1];
  }
}

// kQNoClip: the block-scale rule of Q quantised in the prologue, a template
// parameter rather than a kernel argument (reading the rule there at run time
// cost about 3% of the whole kernel's time on the Qwen3-8B-shaped layer).
template <int D, bool kCausal, bool kDirect, bool kQNoClip>
__global__ __launch_bounds__(256, prefill_min_blocks<D>()) void attn_prefill_kernel(
    AttnArgs a, int ones_scale) {
  using T = PrefillTile<D>;
  constexpr int DB = T::DB, DS = T::DS;
  constexpr int NJ = D / 64;  // QK MFMAs per 32-key tile
  constexpr int NC = D / 32;  // P V channel tiles
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[T::K_RING];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[T::V_RING];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int q_wave0 = qt * kBR + w * 32;
  const int q = q_wave0 + n;
  const int nblk_valid = (L + 31) / 32;
  const int nblk_cap = (a.cap + 31) / 32;

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

  // Prologue loads: K tiles 0, 1, 2 and V tiles 0, 1 (the ring's steady
  // state).  They are issued back to back, so waiting for all of them (and
  // the Q operand) costs little over waiting for K0, V0, K1, and it tells
  // the compiler that no load it knows of is still in flight in the loop.
  // At d = 256, Q rows from the activations are requested first (their
  // quantisation then overlaps the tile loads).
  constexpr bool kQWave = D == 256;
  const bool q_from_raw = a.q_raw != nullptr && q_wave0 < a.Sq;  // uniform
  const int q_nrows = min(32, a.Sq - q_wave0);
  QRaw<D> qr;
  if (kQWave && q_from_raw) q_raw_load<D>(a, bhq * a.Sq + q_wave0, q_nrows, g, lane, qr);
  const TileLanes<D> tl = tile_lanes<D>(w, lane);
  const HeadDescs hd = head_descs<D>(a, bkv, L, nblk_valid, nblk_cap);
  const WaveDst wd = wave_dst<D>(lds_addr(lds_k), lds_addr(lds_v), w);
  const uint32_t vlane = (uint32_t)(w * T::VC_W + lane) * 16u;
  const uint32_t vslane = (uint32_t)(w * T::VS_W + lane) * 4u;
  issue_k<D, 0>(hd, 0, n_tiles, wd, lane, tl);
  issue_v<D, 0>(hd, 0, n_tiles, wd, lane, vlane, vslane);
  issue_k<D, 1>(hd, 1, n_tiles, wd, lane, tl);
  issue_v<D, 1>(hd, 1, n_tiles, wd, lane, vlane, vslane);
  issue_k<D, 2>(hd, 2, n_tiles, wd, lane, tl);
  // The first step's deferred P V (of "tile -1", P = 0) reads V stage 3:
  // give it finite scales.
  for (int i = tid; i < 2 * D; i += 256) lds_v[3 * T::V_BYTES + T::VS_OFF + i] = 0;

  // Q operand (B of S^T = K Q^T): query q, K blocks of 32 along d; its scale
  // bytes packed so that MFMA j reads byte 2*(j%2) of word j/2 (raw words
  // here, shifted for the lane's half once the loads have landed).
  uint4 qa[NJ];
  uint32_t qsw_raw[(NJ + 1) / 2];
  if (kQWave && q_from_raw) {
    // staging: K stage 3 (waves 0, 1) and V stage 2 (waves 2, 3), which no
    // load writes before the first step
    static_assert(2 * QRaw<D>::STAGE <= T::K_BYTES, "Q staging: K stage 3");
    static_assert(2 * QRaw<D>::STAGE <= T::V_BYTES + T::VS_OFF, "Q staging: V stage 2");
    uint8_t* stg = (w < 2 ? lds_k + 3 * T::K_BYTES : lds_v + 2 * T::V_BYTES) + (w & 1) * QRaw<D>::STAGE;
    constexpr uint32_t kQB = kQNoClip ? kScaleBiasNoClip : kScaleBiasOcp;
    if (a.q_raw_bf16) {
      if (a.smooth)
        q_raw_quantise<D, true, true, kQB>(qr, q_nrows, lane, n, h, stg, qa, qsw_raw);
      else
        q_raw_quantise<D, true, false, kQB>(qr, q_nrows, lane, n, h, stg, qa, qsw_raw);
    } else {
      if (a.smooth)
        q_raw_quantise<D, false, true, kQB>(qr, q_nrows, lane, n, h, stg, qa, qsw_raw);
      else
        q_raw_quantise<D, false, false, kQB>(qr, q_nrows, lane, n, h, stg, qa, qsw_raw);
    }
  } else if (!kQWave && q < a.Sq && a.q_raw) {
    constexpr uint32_t kQB = kQNoClip ? kScaleBiasNoClip : kScaleBiasOcp;
    const int64_t qrow = bhq * a.Sq + q;
    if (a.q_raw_bf16) {
      if (a.smooth)
        quantise_q_lane<D, true, true, kQB>(a, qrow, g, h, qa, qsw_raw);
      else
        quantise_q_lane<D, true, false, kQB>(a, qrow, g, h, qa, qsw_raw);
    } else {
      if (a.smooth)
        quantise_q_lane<D, false, true, kQB>(a, qrow, g, h, qa, qsw_raw);
      else
        quantise_q_lane<D, false, false, kQB>(a, qrow, g, h, qa, qsw_raw);
    }
  } else if (q < a.Sq) {
    const uint8_t* qc = a.q_codes + (bhq * a.Sq + q) * DB;
    const uint8_t* qsc = a.q_scales + (bhq * a.Sq + q) * DS;
#pragma unroll
    for (int j = 0; j < NJ; j++) qa[j] = *reinterpret_cast<const uint4*>(qc + 32 * j + 16 * h);
#pragma unroll
    for (int j = 0; j < NJ; j += 2) {
      if constexpr (DS == 2)
        qsw_raw[j / 2] = *reinterpret_cast<const uint16_t*>(qsc);
      else
        qsw_raw[j / 2] = reinterpret_cast<const uint32_t*>(qsc)[j >> 1];
    }
  } else {
#pragma unroll
    for (int j = 0; j < NJ; j++) qa[j] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < NJ; j += 2) qsw_raw[j / 2] = 0;
  }
  HIFA4_WAIT_VMCNT(0);
  __syncthreads();
  int qsw[(NJ + 1) / 2];
#pragma unroll
  for (int j = 0; j < NJ; j += 2) qsw[j / 2] = (int)(qsw_raw[j / 2] >> (8 * h));

  // The lane's K operand offsets within a stage (row 32t + n, chunk 2j + h).
  uint32_t koff[2][NJ];
#pragma unroll
  for (int t = 0; t < 2; t++)
#pragma unroll
    for (int j = 0; j < NJ; j++) {
      const int R = 32 * t + n;
      koff[t][j] = (uint32_t)(R * DB + (((2 * j + h) ^ k_swz<D>(R)) * 16));
    }

  const uint32_t one_bits = n == 0 ? 0x22222222u : 0u;  // E2M1 1.0 in every nibble of row 0
  const uint4 ones = make_uint4(one_bits, one_bits, one_bits, one_bits);
  const float c = a.sm_log2;

  float m_run = -INFINITY;
  uint4 pk = make_uint4(0, 0, 0, 0);
  v16f acc[NC];
#pragma unroll
  for (int cc = 0; cc < NC; cc++) acc[cc] = v16f{};
  v16f accl = v16f{};
  // P_hat of the previous tile, whose P V MFMAs run during this step
  uint4 pend_p = make_uint4(0, 0, 0, 0);
  int pend_s = 127;

  // [acc | l] += P_hat [V | 1] for one tile.
  auto pv_mfma = [&](const VOps<D>& vo, const uint4& p, int ps) {
#pragma unroll
    for (int cc = 0; cc < NC; cc++) acc[cc] = mfma_fp4_32x32x64(vo.va[cc], p, acc[cc], vo.vs[cc], ps);
    if constexpr (!kDirect) accl = mfma_fp4_32x32x64(ones, p, accl, ones_scale, ps);
  };
  // non-reordered normaliser (the sum of the fp32 P), in the running frame
  float l_direct = 0.0f;

  // One pipeline step on tile kt, RP = kt mod 4 (ring slot, a compile-time
  // constant: every LDS address is a per-lane base plus an immediate).
  // Scores of tile kt are in (c0, c1); the next tile's go to (n0r, n1r).
  //   1. LDS reads: K operands of tile kt+1, V operands of tile kt-1;
  //   2. loads of K tile kt+3 and V tile kt+2 into the ring;
  //   3. max phase of tile kt (running max, rescale factor);
  //   4. one block with the Q K^T MFMAs of tile kt+1, the P V MFMAs of tile
  //      kt-1 (its P_hat was packed last step) and the exponentials and
  //      packing of tile kt, interleaved so the matrix core works while
  //      the vector ALU does;
  //   5. rescale of the accumulators (after tile kt-1's P V: frames match);
  //   6. wait for the loads issued last step, barrier.
  // The core block has no branches: a wave whose rows see no key of tile kt
  // masks all its scores (P = 0, the running max stays), and the products
  // of a tile that does not exist read finite stale LDS and are discarded.
  auto step = [&](auto ring, int kt, v16f& c0, v16f& c1, v16f& n0r, v16f& n1r) {
    constexpr int RP = decltype(ring)::value;
    constexpr int NS = T::STAGES;
    const int n0 = kt * kBN;
    const bool do_sm = n0 < wave_end;  // uniform per wave
    KOps<D> ko;
    qk_load<D>(lds_k + ((RP + 1) % NS) * T::K_BYTES, koff, n, h, ko);
    VOps<D> vo;
    v_load<D>(lds_v + ((RP + NS - 1) % NS) * T::V_BYTES, n, h, vo);
    issue_k<D, (RP + 3) % NS>(hd, kt + 3, n_tiles, wd, lane, tl);
    issue_v<D, (RP + 2) % NS>(hd, kt + 2, n_tiles, wd, lane, vlane, vslane);

    if (!do_sm || n0 + kBN > wave_full)
      mask_scores(c0, c1, n0 + 32 * h, do_sm ? row_lim : 0);
    SoftmaxMax sx = softmax_max(c0, c1, m_run, c, a.tau);
    // Order anchors (empty asm, no instructions): the products below may
    // not be hoisted above the max phase, and the rescale test may not be
    // hoisted above the exponentials; otherwise the MFMAs end up clustered
    // instead of interleaved with the vector work.
    asm volatile("" : "+v"(qa[0].x), "+v"(pend_p.x) : "v"(sx.m_use));
    __builtin_amdgcn_sched_barrier(0);
    // Wave priority 1 from here to the end of the rescale: of the two
    // workgroups sharing a SIMD, the wave in its product block issues first
    // and the other fills the gaps (measured: 7 % faster than equal priority).
    __builtin_amdgcn_s_setprio(1);

    qk_mfma<D>(ko, qa, qsw, n0r, n1r);
    pv_mfma(vo, pend_p, pend_s);
    SoftmaxStep st = softmax_exp(c0, c1, sx, c, a.p_bias, pk);
    if constexpr (kDirect) l_direct = __builtin_fmaf(l_direct, st.alpha, row_sum_p(c0, c1));
#pragma unroll
    for (int i = 0; i < NJ * 2 + NC + (kDirect ? 0 : 1); i++) {
      // one MFMA, then a few VALU: ten for d <= 128 (9 MFMAs a step), three for
      // d = 256 (17 MFMAs; measured 365 -> 356 us on the Gemma2 shape)
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, D == 256 ? 3 : 10, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // ... and the Q K^T products may not sink past this step's barrier into
    // the next step, where the max phase would wait for them.
    asm volatile("" : "+v"(st.alpha), "+v"(n0r[0]), "+v"(n1r[0])
                 : "v"(st.p_codes.x), "v"(st.p_codes.y), "v"(st.p_codes.z), "v"(st.p_codes.w));

    // rescale only when some row's max moved (multiplying by 1 is exact); on
    // the first tile the accumulators are still zero
    if (kt != 0 && __any(st.alpha != 1.0f)) {
#pragma unroll
      for (int cc = 0; cc < NC; cc++) acc[cc] *= st.alpha;
      accl[0] *= st.alpha;
    }
    pend_p = st.p_codes;
    pend_s = st.p_scale;
    __builtin_amdgcn_s_setprio(0);
    // K tile kt+2 and V tile kt (issued one and two steps ago) have landed;
    // this step's loads stay in flight.
    HIFA4_WAIT_VMCNT(T::N_LOADS);
    __syncthreads();
  };

  // Two-phase step (d = 256) on tile kt, RP = kt mod 4; the scores of tile kt
  // are in (s0, s1):
  //   1. loads of K tile kt+3 and V tile kt+2 into the ring (as above);
  //   2. softmax of tile kt: mask, running max, exponentials, P_hat (vector ALU);
  //   3. rescale of the accumulators (rarely: only when some row's frame moved);
  //   4. at wave priority 1, the products: [acc | l] += P_hat [V | 1] for tile kt
  //      and the next tile's scores, S = Q K^T of tile kt+1, into (s0, s1), with
  //      each operand read from LDS just before its MFMA;
  //   5. wait for the loads issued last step, barrier.
  // Same ring, waits and LDS layouts as the one-phase step: step kt reads V
  // tile kt (landed: issued two steps earlier) and K tile kt+1.
  //
  // Registers: the K-operand offsets of the second 32-key tile are those of
  // the first plus a constant (with chunk pairs j and j ^ 2 swapped at
  // d = 256, see KX), and the normaliser is kept as one
  // value per lane (l2, lanes of row 0 of the ones-column product), the
  // product itself starting from zero every step: the live state fits two
  // waves per SIMD without spills.
  float l2 = 0.0f;
  // The lane's V operand and V scale bytes in ring stage 0 (channel tile 0):
  // every other stage and channel tile is a compile-time offset from them,
  // which the LDS reads take as immediates (the V ring lies above 64 KB of LDS
  // at d = 256, out of reach of an immediate offset from address 0; written
  // as one expression per read, the compiler had kept one address register
  // per channel tile and added the stage base each step).
  const uint8_t* v_op0 = lds_v + (h * D + n) * 16;
  const uint8_t* v_sc0 = lds_v + T::VS_OFF + h * D + n;
  auto step2 = [&](auto ring, int kt, v16f& s0, v16f& s1) {
    // row 32 + n's chunk swizzle is row n's XOR 4 at d = 256 and the same at
    // d = 64 / 128 (k_swz), so its chunk 2j + h is row n's chunk 2 (j ^ KX) + h
    constexpr int KX = D == 256 ? 2 : 0;
    constexpr int RP = decltype(ring)::value;
    constexpr int NS = T::STAGES;
    const int n0 = kt * kBN;
    const bool do_sm = n0 < wave_end;  // uniform per wave
    issue_k<D, (RP + 3) % NS>(hd, kt + 3, n_tiles, wd, lane, tl);
    issue_v<D, (RP + 2) % NS>(hd, kt + 2, n_tiles, wd, lane, vlane, vslane);

    // A wave whose rows see no key of tile kt sees none of the later tiles
    // either (the causal limit is fixed and kt grows): its P would be 0, the
    // products would add exact zeros and the next scores are never used, so
    // it only keeps the ring's loads and barriers in step with the others.
    // Same bits; the other waves on the SIMD get its issue slots (Gemma2 /
    // Llama-3.1-8B-shaped layers 211.8 / 150.8 -> 208.1 / 147.2 us).
    if (do_sm) {
      if (n0 + kBN > wave_full) mask_scores(s0, s1, n0 + 32 * h, row_lim);
      const SoftmaxMax sx = softmax_max<true>(s0, s1, m_run, c, a.tau);
      // the packing register: the converts overwrite every byte of it, so it
      // starts from whatever the registers hold (no zeroing moves)
      uint4 pz;
      asm volatile("" : "=v"(pz.x), "=v"(pz.y), "=v"(pz.z), "=v"(pz.w));
      const SoftmaxStep st = softmax_exp(s0, s1, sx, c, a.p_bias, pz);
      if constexpr (kDirect) l_direct = __builtin_fmaf(l_direct, st.alpha, row_sum_p(s0, s1));
      if (kt != 0 && sx.moved) {
#pragma unroll
        for (int cc = 0; cc < NC; cc++) acc[cc] *= st.alpha;
        l2 *= st.alpha;
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int cc = 0; cc < NC; cc++) {
        const uint4 va = *reinterpret_cast<const uint4*>(v_op0 + RP * T::V_BYTES + cc * 512);
        const int vs = v_sc0[RP * T::V_BYTES + cc * 32];
        acc[cc] = mfma_fp4_32x32x64(va, st.p_codes, acc[cc], vs, st.p_scale);
      }
      if constexpr (!kDirect) {
        const v16f lt = mfma_fp4_32x32x64(ones, st.p_codes, v16f{}, ones_scale, st.p_scale);
        l2 += lt[0];
      }
      const uint8_t* kbuf = lds_k + ((RP + 1) % NS) * T::K_BYTES;
      const uint8_t* ksc = kbuf + T::KS_OFF;
      s0 = v16f{};
      s1 = v16f{};
#pragma unroll
      for (int j = 0; j < NJ; j++) {
        const uint4 k0 = *reinterpret_cast<const uint4*>(kbuf + koff[0][j]);
        const uint4 k1 = *reinterpret_cast<const uint4*>(kbuf + 32 * DB + koff[0][j ^ KX]);
        const int ks0 = k_scale_word<DS>(ksc + n * T::KSS, j, h);
        const int ks1 = k_scale_word<DS>(ksc + (32 + n) * T::KSS, j, h);
        if (j % 2 == 0) {
          s0 = mfma_fp4_sel<0>(k0, qa[j], s0, ks0, qsw[j / 2]);
          s1 = mfma_fp4_sel<0>(k1, qa[j], s1, ks1, qsw[j / 2]);
        } else {
          s0 = mfma_fp4_sel<2>(k0, qa[j], s0, ks0, qsw[j / 2]);
          s1 = mfma_fp4_sel<2>(k1, qa[j], s1, ks1, qsw[j / 2]);
        }
      }
      // the operand reads run ahead of the MFMAs: six at the start, then two
      // more before each MFMA (218 -> 208 us on the Gemma2 shape, same bits;
      // eight or ten ahead spill)
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
      for (int i = 0; i < NC + 1 + 2 * NJ; i++) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
    }
    // K tile kt+2 and V tile kt+1 (issued one and two steps ago) have landed;
    // this step's loads stay in flight.
    HIFA4_WAIT_VMCNT(T::N_LOADS);
    __syncthreads();
  };

  // a wave whose rows see no key never computes (sa0, sa1): zeros, then masked
  v16f sa0{}, sa1{}, sb0, sb1;
  if (0 < wave_end) {
    KOps<D> ko;
    qk_load<D>(lds_k, koff, n, h, ko);
    qk_mfma<D>(ko, qa, qsw, sa0, sa1);
  }
  using R0 = std::integral_constant<int, 0>;
  using R1 = std::integral_constant<int, 1>;
  using R2 = std::integral_constant<int, 2>;
  using R3 = std::integral_constant<int, 3>;
  if constexpr (prefill_two_phase<D>()) {
    (void)step;
    for (int kt = 0; kt < n_tiles; kt += 4) {
      step2(R0{}, kt, sa0, sa1);
      if (kt + 1 >= n_tiles) break;
      step2(R1{}, kt + 1, sa0, sa1);
      if (kt + 2 >= n_tiles) break;
      step2(R2{}, kt + 2, sa0, sa1);
      if (kt + 3 >= n_tiles) break;
      step2(R3{}, kt + 3, sa0, sa1);
    }
  } else {
    (void)step2;
    for (int kt = 0; kt < n_tiles; kt += 4) {
      // The loop header is 64-byte aligned (build flags); three 4-byte nops
      // put the body at byte 12 of its line.  This step's speed depended on
      // that position when d = 128 still ran it (16 positions 0, 4, .., 60 on
      // the Qwen3-8B / Llama-3.1-8B-shaped layers: bodies starting at 12 mod 16
      // ran at 69-71 / 163-165 us, at 0 mod 16 at 75-82 / 167-170 us, for the
      // same instructions); the two-phase loop showed no such dependence at
      // d = 256 (209-212 us over all 16 positions).
      asm volatile("s_nop 0\n\ts_nop 0\n\ts_nop 0");
      step(R0{}, kt, sa0, sa1, sb0, sb1);
      if (kt + 1 >= n_tiles) break;
      step(R1{}, kt + 1, sb0, sb1, sa0, sa1);
      if (kt + 2 >= n_tiles) break;
      step(R2{}, kt + 2, sa0, sa1, sb0, sb1);
      if (kt + 3 >= n_tiles) break;
      step(R3{}, kt + 3, sb0, sb1, sa0, sa1);
    }
    // the last tile's P V
    if (n_tiles > 0) {
      VOps<D> vo;
      v_load<D>(lds_v + ((n_tiles - 1) % T::STAGES) * T::V_BYTES, n, h, vo);
      pv_mfma(vo, pend_p, pend_s);
    }
  }
  // No load may still be writing this workgroup's LDS when it exits; at
  // d = 256 the rings take the output tiles once every wave is past its last
  // ring read.
  HIFA4_WAIT_VMCNT(0);
  if constexpr (!T::OUT_OWN) __syncthreads();

  // Wave priority 2 for the epilogue: a finishing item frees its slot sooner when
  // the other workgroup on the SIMD is in its priority-1 product block (measured:
  // 1.4 % faster on the Qwen3-8B shape, 0.2-0.4 % on the Llama and Gemma2 shapes).
  __builtin_amdgcn_s_setprio(2);
  // ---- epilogue: O = acc / l, LSE = m ln2 + ln l
  // The lane index again, from the lane-count instruction rather than from
  // threadIdx: the thread id would otherwise stay live across the loop only for
  // these uses, and at d = 256 it was the one register spilled (a 4-byte store
  // per lane, 2 MiB of the Gemma2-shaped launch's writes).
  const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int n_e = lane_e & 31, h_e = lane_e >> 5;
  const float lsum = kDirect ? l_direct : __shfl(prefill_two_phase<D>() ? l2 : accl[0], n_e);
  // rows of this wave inside the sequence; the lane's row is row0 + n (written
  // without q, which would otherwise stay live across the loop and spill at
  // d = 256)
  const int nrows = min(32, a.Sq - q_wave0);
  const int64_t row0 = bhq * a.Sq + q_wave0;
  if (nrows > 0) {
    const float inv = n_e < nrows && lsum > 0.0f ? 1.0f / lsum : 0.0f;
    uint8_t* stage;
    if constexpr (T::OUT_OWN) {
      __shared__ __attribute__((aligned(16))) uint8_t lds_o[4 * T::OUT_TILE];
      stage = lds_o + w * T::OUT_TILE;
    } else {
      stage = (w < 2 ? lds_k : lds_v) + (w & 1) * T::OUT_TILE;
    }
    // the output type is chosen once per wave, not per element
    if (a.out_fp16)
      write_out<NC, true>(a, row0, nrows, n_e, h_e, lane_e, acc, inv, stage);
    else
      write_out<NC, false>(a, row0, nrows, n_e, h_e, lane_e, acc, inv, stage);
  }
  if (n_e < nrows && a.lse && h_e == 0)
    a.lse[row0 + n_e] = lsum > 0.0f ? m_run * kLn2 + logf(lsum) : -INFINITY;
}

// ---------------------------------------------------------------------------
// Decode (Sq == 1), split-K over a balanced schedule (below).  A wave runs
// the online softmax of one run of key tiles of one (sequence, KV head)
// against the G query heads of the group (the MFMA's 32 query columns, G
// used) and writes one partial (m, l, acc[d]) per query head; the merge
// kernel combines the runs of a pair with the log-sum-exp rule.
//
// Decode reads every K / V byte once, so it is bound by how many bytes are
// in flight.  Each wave streams its tiles through a private LDS ring with
// memory -> LDS buffer loads (no registers held by loads in flight): while
// tile t is computed from registers, the ring's other stages are loading, and
// tile t's stage is refilled as soon as its operands are in registers.  The
// K layout in a stage is the prefill one (rows in MFMA read order, swizzled
// chunks), so the operand reads are shared with prefill.  Keys past the
// sequence read zeros (descriptor range) and are masked.
// ---------------------------------------------------------------------------
template <int D>
struct DecStage {
  using T = PrefillTile<D>;
  static constexpr int BYTES = T::K_BYTES + T::V_BYTES;  // K then V of one 64-key tile
  static constexpr int KC_I = kBN * T::DB / 1024;        // 1 KB K code loads per tile
  static constexpr int VC_I = 2 * D * 16 / 1024;         // 1 KB V code loads per tile
  static constexpr int KS_I = T::DS == 8 ? 2 : 1;        // K scale loads (2 or 4 bytes a lane)
  static constexpr int VS_I = D == 256 ? 2 : 1;          // V scale loads (4 bytes a lane)
  static constexpr int N_LOADS = KC_I + VC_I + KS_I + VS_I;
  static_assert(2 * N_LOADS < 64, "vmcnt counts up to 63");
};

// s_waitcnt immediate for vmcnt(n), other counters untouched (gfx9 encoding:
// vmcnt bits [3:0] and [15:14]).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 0xF) | ((n >> 4) << 14); }
// lgkmcnt(0) alone.
constexpr int kLgkm0 = 0xC07F;

// Per-lane source offsets of a whole tile's loads (loop invariant).
template <int D>
struct DecLanes {
  uint32_t kc[DecStage<D>::KC_I];
  uint32_t ks[DecStage<D>::KS_I];
};

template <int D>
__device__ __forceinline__ DecLanes<D> dec_lanes(int lane) {
  using T = PrefillTile<D>;
  DecLanes<D> dl;
#pragma unroll
  for (int i = 0; i < DecStage<D>::KC_I; i++) {
    const int b = 64 * i + lane;  // chunk index in LDS order
    const int R = b / T::NCH, pos = b % T::NCH;
    dl.kc[i] = (uint32_t)(perm_row(R >> 5, R & 31) * T::DB + ((pos ^ k_swz<D>(R)) * 16));
  }
#pragma unroll
  for (int i = 0; i < DecStage<D>::KS_I; i++) {
    // one row per lane (two lanes per row for 8-byte rows)
    const int R = T::DS == 8 ? 32 * i + (lane >> 1) : lane;
    dl.ks[i] = (uint32_t)(perm_row(R >> 5, R & 31) * T::DS + (T::DS == 8 ? 4 * (lane & 1) : 0));
  }
  return dl;
}

// Issue the loads of the 64-key tile starting at key n0 (live) into the
// stage at LDS address `st`; a dead tile reads nothing but still issues.
template <int D>
__device__ __forceinline__ void dec_issue(const HeadDescs& hd, int n0, bool live, uint32_t st,
                                          int lane, const DecLanes<D>& dl) {
  using T = PrefillTile<D>;
  using S = DecStage<D>;
  const int soc = live ? n0 * T::DB : kPastEnd;
  const int sos = live ? n0 * T::DS : kPastEnd;
  const int svc = live ? (n0 / 32) * D * 16 : kPastEnd;
  const int svs = live ? (n0 / 32) * D : kPastEnd;
#pragma unroll
  for (int i = 0; i < S::KC_I; i++) load_lds16<0>(hd.kc, dl.kc[i], soc, st + 1024 * i);
#pragma unroll
  for (int i = 0; i < S::KS_I; i++) {
    if constexpr (T::DS == 2)
      load_lds2<0>(hd.ks, dl.ks[i], sos, st + T::KS_OFF);
    else
      load_lds4<0>(hd.ks, dl.ks[i], sos, st + T::KS_OFF + 256 * i);
  }
  const uint32_t sv = st + T::K_BYTES;
#pragma unroll
  for (int i = 0; i < S::VC_I; i++)
    load_lds16<0>(hd.vc, (uint32_t)(1024 * i + 16 * lane), svc, sv + 1024 * i);
#pragma unroll
  for (int i = 0; i < S::VS_I; i++) {
    if (D == 64 && lane >= 32) break;  // 128 scale bytes
    load_lds4<0>(hd.vs, (uint32_t)(256 * i + 4 * lane), svs, sv + T::VS_OFF + 256 * i);
  }
}

// ---------------------------------------------------------------------------
// Split-K schedules.  Pair s = (sequence b, KV head g), s = b * Hkv + g, has
// tiles(L_b) = ceil(L_b / 64) key tiles.  Wave w of the persistent grid takes
// pieces w, w + W, ...; a piece runs the online softmax from a fresh state.
//
// Balanced (decode_chunk == 0): the pairs' tiles laid end to end (sequence
// outer) form one sequence of `total` tiles, cut into pieces of
// decode_piece_tiles(...) tiles, an even share per wave; a piece restarts
// where it crosses into the next pair.  Each (piece, pair) run leaves one
// partial row per query head of the pair at workspace row piece + s, which is
// unique: a later piece never covers an earlier pair.  Where a pair's runs
// start depends on the lengths of the sequences before it.
//
// Per pair (decode_chunk > 0, pt = decode_chunk / 64 tiles): pair s is cut
// from its own key 0 into ceil(tiles / pt) pieces of pt tiles (the last one
// shorter), numbered pair after pair; piece p leaves its partial rows at
// workspace row p.  A pair's runs, and so its result, depend on its own length
// only.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int dec_len(const AttnArgs& a, int b) {
  if (b >= a.B) return 0;
  return a.kv_lens ? min(max(a.kv_lens[b], 0), a.Sk) : a.Sk;
}

__device__ __forceinline__ int dec_tiles(int L) { return (L + kBN - 1) / kBN; }

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Inclusive prefix sum over the lanes of a wave.
__device__ __forceinline__ int wave_scan_i(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Tiles of all pairs, and of the pairs of the sequences before b.
struct DecTotals {
  int total, before;
};

__device__ __forceinline__ DecTotals dec_totals(const AttnArgs& a, int b, int lane) {
  int tot = 0, bef = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int bb = b0 + lane;
    const int nt = dec_tiles(dec_len(a, bb));
    tot += nt;
    bef += bb < b ? nt : 0;
  }
  return {uniform(wave_sum_i(tot) * a.Hkv), uniform(wave_sum_i(bef) * a.Hkv)};
}

// Where a wave stands in the tile sequence: pair (b, g) with L keys and nt
// tiles, and the tile lt within it.
struct DecCursor {
  int b, g, lt, nt, L;
};

// The pair and tile of flattened tile t < total: a wave-parallel search over
// the sequences' tile counts, 64 sequences at a time.
__device__ DecCursor dec_locate(const AttnArgs& a, int t, int lane) {
  DecCursor c{0, 0, 0, 1, 0};
  int base = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int bb = b0 + lane;
    const int L = dec_len(a, bb);
    const int nt = dec_tiles(L);
    const int incl = base + wave_scan_i(nt * a.Hkv, lane);
    const uint64_t hit = __ballot(bb < a.B && incl > t);
    if (hit) {
      const int i = __builtin_ctzll(hit);  // first sequence whose pairs reach past t
      c.b = b0 + i;
      c.L = __shfl(L, i);
      c.nt = __shfl(nt, i);
      const int off = t - (__shfl(incl, i) - c.nt * a.Hkv);
      c.g = off / c.nt;
      c.lt = off - c.g * c.nt;
      break;
    }
    base = __shfl(incl, 63);
  }
  return {uniform(c.b), uniform(c.g), uniform(c.lt), uniform(c.nt), uniform(c.L)};
}

__device__ __forceinline__ int dec_pair_pieces(int nt, int pt) { return (nt + pt - 1) / pt; }

// Per-pair schedule: pieces of all pairs (b_end = B), or of the pairs of the
// sequences before b_end.
__device__ __forceinline__ int dec_pieces_before(const AttnArgs& a, int b_end, int pt, int lane) {
  int tot = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int bb = b0 + lane;
    tot += bb < b_end ? dec_pair_pieces(dec_tiles(dec_len(a, bb)), pt) : 0;
  }
  return uniform(wave_sum_i(tot) * a.Hkv);
}

// Per-pair schedule: the pair of piece p < (all pieces) and the piece's first tile
// within it.
__device__ DecCursor dec_locate_piece(const AttnArgs& a, int p, int pt, int lane) {
  DecCursor c{0, 0, 0, 1, 0};
  int base = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int bb = b0 + lane;
    const int L = dec_len(a, bb);
    const int nt = dec_tiles(L);
    const int np = dec_pair_pieces(nt, pt);
    const int incl = base + wave_scan_i(np * a.Hkv, lane);
    const uint64_t hit = __ballot(bb < a.B && incl > p);
    if (hit) {
      const int i = __builtin_ctzll(hit);  // first sequence whose pieces reach past p
      const int npi = __shfl(np, i);
      c.b = b0 + i;
      c.L = __shfl(L, i);
      c.nt = __shfl(nt, i);
      const int off = p - (__shfl(incl, i) - npi * a.Hkv);
      c.g = off / npi;
      c.lt = (off - c.g * npi) * pt;
      break;
    }
    base = __shfl(incl, 63);
  }
  return {uniform(c.b), uniform(c.g), uniform(c.lt), uniform(c.nt), uniform(c.L)};
}

// The first tile of the next pair that has any (the caller knows one exists).
__device__ __forceinline__ void dec_next_pair(const AttnArgs& a, DecCursor& c) {
  c.lt = 0;
  if (++c.g < a.Hkv) return;
  c.g = 0;
  do {
    ++c.b;
    c.L = dec_len(a, c.b);
    c.nt = dec_tiles(c.L);
  } while (c.nt == 0 && c.b + 1 < a.B);
}

template <int D>
__device__ __forceinline__ HeadDescs dec_descs(const AttnArgs& a, const DecCursor& c) {
  return head_descs<D>(a, (int64_t)c.b * a.Hkv + c.g, c.L, (c.L + 31) / 32, (a.cap + 31) / 32);
}

// Per-wave LDS ring of the decode kernel; the persistent grid has as many
// waves per compute unit as the 160 KB of LDS holds rings (at most eight).
template <int D>
struct DecRing {
  static constexpr int STAGES = D == 64 ? 4 : 2;  // about 35 KB of loads in flight per wave
  static constexpr int BYTES = STAGES * DecStage<D>::BYTES;
  static constexpr int WAVES_PER_CU = 163840 / BYTES < 8 ? 163840 / BYTES : 8;
};
constexpr int kComputeUnits = 256;  // MI355X

// Partial row of one query head: m (log2 units), l, two unused floats, acc[d].
template <int D>
__device__ __forceinline__ void dec_flush(const AttnArgs& a, int prow, int G, int n, int h,
                                          float m_run, float lsum, const v16f* acc) {
  constexpr int NC = D / 32;
  if (n < G) {
    float* row = a.partials + ((int64_t)prow * G + n) * (D + 4);
    if (h == 0) {
      row[0] = m_run;
      row[1] = lsum;
    }
#pragma unroll
    for (int cc = 0; cc < NC; cc++)
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        const int ch = 32 * cc + 8 * g4 + 4 * h;
        *reinterpret_cast<float4*>(row + 4 + ch) =
            make_float4(acc[cc][4 * g4], acc[cc][4 * g4 + 1], acc[cc][4 * g4 + 2], acc[cc][4 * g4 + 3]);
      }
  }
}

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int D, bool kDirect>
__global__ __launch_bounds__(64, DecRing<D>::WAVES_PER_CU / 4) void attn_decode_kernel(AttnArgs a,
                                                                              int ones_scale) {
  using T = PrefillTile<D>;
  using S = DecStage<D>;
  constexpr int NS = DecRing<D>::STAGES;
  constexpr int DB = T::DB, DS = T::DS, NJ = D / 64, NC = D / 32;
  __shared__ __attribute__((aligned(16))) uint8_t ring[NS * S::BYTES];

  const int lane = threadIdx.x;
  const int h = lane >> 5, n = lane & 31;
  const int G = a.Hq / a.Hkv;
  const bool per_pair = a.chunk > 0;
  const int total = dec_totals(a, 0, lane).total;
  const int pt = decode_piece_tiles(a.chunk, a.dec_waves, total);
  const int n_pieces = per_pair ? dec_pieces_before(a, a.B, pt, lane) : (total + pt - 1) / pt;
  if ((int)blockIdx.x >= n_pieces) return;  // uniform per wave

  const DecLanes<D> dl = dec_lanes<D>(lane);
  const uint32_t ring_addr = lds_addr(ring);
  uint32_t koff[2][NJ];
#pragma unroll
  for (int t = 0; t < 2; t++)
#pragma unroll
    for (int j = 0; j < NJ; j++) {
      const int R = 32 * t + n;
      koff[t][j] = (uint32_t)(R * DB + (((2 * j + h) ^ k_swz<D>(R)) * 16));
    }
  const uint32_t one_bits = n == 0 ? 0x22222222u : 0u;
  const uint4 ones = make_uint4(one_bits, one_bits, one_bits, one_bits);
  const float c = a.sm_log2;

  // Q operand of a pair: column n is query head g*G + n (zero for n >= G).
  uint4 qa[NJ];
  uint32_t qsw_raw[(NJ + 1) / 2];
  int qsw[(NJ + 1) / 2];
  auto load_q = [&](const DecCursor& cur) {
    if (n < G) {
      const int64_t row = (int64_t)cur.b * a.Hq + cur.g * G + n;  // Sq == 1
      const uint8_t* qc = a.q_codes + row * DB;
      const uint8_t* qsc = a.q_scales + row * DS;
#pragma unroll
      for (int j = 0; j < NJ; j++) qa[j] = *reinterpret_cast<const uint4*>(qc + 32 * j + 16 * h);
#pragma unroll
      for (int j = 0; j < NJ; j += 2) {
        if constexpr (DS == 2)
          qsw_raw[j / 2] = *reinterpret_cast<const uint16_t*>(qsc);
        else
          qsw_raw[j / 2] = reinterpret_cast<const uint32_t*>(qsc)[j >> 1];
      }
    } else {
#pragma unroll
      for (int j = 0; j < NJ; j++) qa[j] = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < NJ; j += 2) qsw_raw[j / 2] = 0;
    }
  };
  auto shift_q = [&]() {
#pragma unroll
    for (int j = 0; j < NJ; j += 2) qsw[j / 2] = (int)(qsw_raw[j / 2] >> (8 * h));
  };

  uint4 pk = make_uint4(0, 0, 0, 0);
  for (int piece = blockIdx.x; piece < n_pieces; piece += gridDim.x) {
    // [t_beg, t_end): the piece's tiles (flattened indices for the balanced
    // schedule, counted from 0 within its one pair for the per-pair schedule)
    int t_beg, t_end;
    DecCursor cc;  // pair of the tile being computed
    if (per_pair) {
      cc = dec_locate_piece(a, piece, pt, lane);
      t_beg = 0;
      t_end = min(pt, cc.nt - cc.lt);
    } else {
      t_beg = piece * pt;
      t_end = min(total, t_beg + pt);
      cc = dec_locate(a, t_beg, lane);
    }
    DecCursor ic = cc;                           // pair of the next tile to load
    HeadDescs hd = dec_descs<D>(a, ic);
    int ti = t_beg;                              // next tile to load
    // Load tile ti (nothing past the piece) into the stage at LDS address st.
    auto issue = [&](uint32_t st) {
      const bool live = ti < t_end;
      dec_issue<D>(hd, ic.lt * kBN, live, st, lane, dl);
      if (live && ti + 1 < t_end && ++ic.lt == ic.nt) {
        dec_next_pair(a, ic);
        hd = dec_descs<D>(a, ic);
      }
      ++ti;
    };
#pragma unroll
    for (int s = 0; s < NS; s++) issue(ring_addr + s * S::BYTES);
    load_q(cc);
    // Q and the first tiles: the compiler then knows no load of its own is
    // in flight in the loop.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    shift_q();

    float m_run = -INFINITY;
    float l_direct = 0.0f;  // non-reordered normaliser (sum of the fp32 P)
    v16f acc[NC];
#pragma unroll
    for (int k = 0; k < NC; k++) acc[k] = v16f{};
    v16f accl = v16f{};

    // One 64-key step on tile t, held in stage SP.
    auto step = [&](auto stage, int t) {
      constexpr int SP = decltype(stage)::value;
      const uint8_t* st = ring + SP * S::BYTES;
      // tile t has landed; the NS - 1 tiles after it may still be loading
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 1) * S::N_LOADS));
      KOps<D> ko;
      qk_load<D>(st, koff, n, h, ko);
      VOps<D> vo;
      v_load<D>(st + T::K_BYTES, n, h, vo);
      v16f s_lo, s_hi;
      qk_mfma<D>(ko, qa, qsw, s_lo, s_hi);
      // every read of this stage is done: refill it
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      issue(ring_addr + SP * S::BYTES);

      const bool pair_end = cc.lt + 1 == cc.nt;
      if (pair_end && (cc.L & (kBN - 1))) mask_scores(s_lo, s_hi, cc.lt * kBN + 32 * h, cc.L);
      const SoftmaxStep sm = softmax_step(s_lo, s_hi, m_run, c, a.tau, a.p_bias, pk);
      if constexpr (kDirect) l_direct = __builtin_fmaf(l_direct, sm.alpha, row_sum_p(s_lo, s_hi));
      if (__any(sm.alpha != 1.0f)) {
#pragma unroll
        for (int k = 0; k < NC; k++) acc[k] *= sm.alpha;
        accl[0] *= sm.alpha;
      }
#pragma unroll
      for (int k = 0; k < NC; k++)
        acc[k] = mfma_fp4_32x32x64(vo.va[k], sm.p_codes, acc[k], vo.vs[k], sm.p_scale);
      if constexpr (!kDirect)
        accl = mfma_fp4_32x32x64(ones, sm.p_codes, accl, ones_scale, sm.p_scale);

      if (pair_end || t + 1 == t_end) {
        dec_flush<D>(a, per_pair ? piece : piece + cc.b * a.Hkv + cc.g, G, n, h, m_run,
                     kDirect ? l_direct : __shfl(accl[0], n), acc);
        m_run = -INFINITY;
        l_direct = 0.0f;
#pragma unroll
        for (int k = 0; k < NC; k++) acc[k] = v16f{};
        accl = v16f{};
        if (t + 1 < t_end) {
          dec_next_pair(a, cc);
          load_q(cc);
        }
        // the partial stores, Q and the ring's loads in flight: the step-start
        // wait counts only ring loads
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        shift_q();
      } else {
        ++cc.lt;
      }
    };
    for (int t = t_beg; t < t_end; t += NS)
      static_for<NS>([&](auto sp) {
        if (t + decltype(sp)::value < t_end) step(sp, t + decltype(sp)::value);
      });
  }
}

// Log-sum-exp merge of a pair's runs: one wave per (sequence, query head),
// lane i owning channels i, i + 64, ...  One pass over the runs, U at a time:
// the U rows (m, l, acc) are loaded together, then folded into the running
// (M, l, o) with the online rule, so a pair with at most U runs costs one
// round trip to memory.
template <int D>
__global__ __launch_bounds__(256) void attn_decode_merge_kernel(AttnArgs a) {
  constexpr int CPL = (D + 63) / 64;  // channels per lane
  constexpr int U = 16;               // runs per round
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);  // b * Hq + hq
  if (row >= (int64_t)a.B * a.Hq) return;
  const int b = (int)(row / a.Hq), hq = (int)(row % a.Hq);
  const int G = a.Hq / a.Hkv, g = hq / G, hh = hq % G;
  const DecTotals tt = dec_totals(a, b, lane);
  const int nt = dec_tiles(dec_len(a, b));
  const int64_t stride = (int64_t)G * (D + 4);  // between the rows of consecutive pieces
  int nc = 0;
  const float* part = a.partials;
  if (nt > 0) {
    const int pt = decode_piece_tiles(a.chunk, a.dec_waves, tt.total);
    int64_t row0;  // the pair's first partial row; its runs' rows follow it
    if (a.chunk > 0) {
      nc = dec_pair_pieces(nt, pt);
      row0 = dec_pieces_before(a, b, pt, lane) + g * nc;
    } else {
      const int first = tt.before + g * nt;  // flattened index of the pair's first tile
      const int j0 = first / pt;
      nc = (first + nt - 1) / pt - j0 + 1;
      row0 = j0 + b * a.Hkv + g;
    }
    part += (row0 * G + hh) * (D + 4);
  }
  float M = -INFINITY, lsum = 0.0f;
  float o[CPL];
#pragma unroll
  for (int j = 0; j < CPL; j++) o[j] = 0.0f;
  for (int i0 = 0; i0 < nc; i0 += U) {
    float mu[U], lu[U], x[U][CPL];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const bool ok = i0 + u < nc;
      const float* pr = part + (int64_t)(ok ? i0 + u : 0) * stride;
      const float2 ml = *reinterpret_cast<const float2*>(pr);
      mu[u] = ok ? ml.x : -INFINITY;
      lu[u] = ml.y;
#pragma unroll
      for (int j = 0; j < CPL; j++) {
        const int ch = lane + 64 * j;
        x[u][j] = ch < D ? pr[4 + ch] : 0.0f;
      }
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < U; u++) Mn = fmaxf(Mn, mu[u]);
    const float keep = M == -INFINITY ? 0.0f : fast_exp2(M - Mn);
    lsum *= keep;
#pragma unroll
    for (int j = 0; j < CPL; j++) o[j] *= keep;
#pragma unroll
    for (int u = 0; u < U; u++) {
      const float w = mu[u] == -INFINITY ? 0.0f : fast_exp2(mu[u] - Mn);
      lsum += w * lu[u];
#pragma unroll
      for (int j = 0; j < CPL; j++) o[j] += w * x[u][j];
    }
    M = Mn;
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

template <int D, bool kQNoClip>
void launch_prefill_rule(const AttnArgs& a, dim3 g, dim3 b, hipStream_t stream) {
  if (a.causal && !a.direct_l)
    hipLaunchKernelGGL((attn_prefill_kernel<D, true, false, kQNoClip>), g, b, 0, stream, a,
                       kScaleOne);
  else if (!a.direct_l)
    hipLaunchKernelGGL((attn_prefill_kernel<D, false, false, kQNoClip>), g, b, 0, stream, a,
                       kScaleOne);
  else if (a.causal)
    hipLaunchKernelGGL((attn_prefill_kernel<D, true, true, kQNoClip>), g, b, 0, stream, a,
                       kScaleOne);
  else
    hipLaunchKernelGGL((attn_prefill_kernel<D, false, true, kQNoClip>), g, b, 0, stream, a,
                       kScaleOne);
}

template <int D>
hipError_t launch_prefill_d(const AttnArgs& a, hipStream_t stream) {
  const int n_qt = (a.Sq + kBR - 1) / kBR;
  const int64_t grid = (int64_t)n_qt * a.B * a.Hq;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid), b(256);
  // the no-clip Q instances only matter when Q is quantised in the prologue
  if (a.q_raw && a.q_bias == kScaleBiasNoClip)
    launch_prefill_rule<D, true>(a, g, b, stream);
  else
    launch_prefill_rule<D, false>(a, g, b, stream);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const AttnArgs& a, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  if (a.Hq / a.Hkv > 32) return hipErrorNotSupported;  // one MFMA column per query head
  if (a.direct_l)
    hipLaunchKernelGGL((attn_decode_kernel<D, true>), dim3(a.dec_waves), dim3(64), 0, stream, a,
                       kScaleOne);
  else
    hipLaunchKernelGGL((attn_decode_kernel<D, false>), dim3(a.dec_waves), dim3(64), 0, stream, a,
                       kScaleOne);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)a.B * a.Hq;
  hipLaunchKernelGGL(attn_decode_merge_kernel<D>, dim3((unsigned)((rows + kWaves - 1) / kWaves)),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int attn_block_n(int) { return kBN; }
int attn_decode_waves(int d) {
  switch (d) {
    case 64: return kComputeUnits * DecRing<64>::WAVES_PER_CU;
    case 128: return kComputeUnits * DecRing<128>::WAVES_PER_CU;
    case 256: return kComputeUnits * DecRing<256>::WAVES_PER_CU;
  }
  return kComputeUnits;
}

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
