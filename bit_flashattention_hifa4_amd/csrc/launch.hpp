// launch.hpp -- internal interface between the C ABI (api.cpp) and the kernel
// translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hifa4 {

// Block-scale rules, as the bias the kernels add to a block maximum's fp32 bit
// pattern before taking its exponent field: the OCP MX shared exponent, or the
// no-clip one (one higher wherever the OCP exponent would saturate an element).
constexpr uint32_t kScaleBiasOcp = 0u;
constexpr uint32_t kScaleBiasNoClip = 0x003FFFFFu;

struct QuantizeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* smooth;
  uint8_t* q_codes;
  uint8_t* q_scales;
  uint8_t* k_codes;
  uint8_t* k_scales;
  uint8_t* v_codes;
  uint8_t* v_scales;
  int B, Hq, Hkv, Sq, Sk, d, cap;
  int64_t blocks_q, blocks_k;  // 32-element row blocks
  int64_t wg_q, wg_k;          // filled by the launcher
  int64_t items_v;             // (channel pair, 32-token block) items; filled by the launcher
  const float* rope_cos;       // rotate-half RoPE tables [n_pos][d/2] for Q and K, or null
  const float* rope_sin;
  int q_pos0, k_pos0;          // position of token 0 of Q / K in the tables
  uint32_t q_bias, k_bias, v_bias;  // block-scale rule of each output (kScaleBias*)
};

hipError_t launch_quantize_qkv(QuantizeArgs a, bool bf16, hipStream_t stream);

// KV-cache append: n_new tokens per sequence at positions lens[b] ...
struct AppendArgs {
  const uint16_t* q;      // [B][Hq][n_new][d] or null
  const uint16_t* k;      // [B][Hkv][n_new][d]
  const uint16_t* v;      // [B][Hkv][n_new][d]
  const float* smooth;    // [Hkv][d] or null
  const float* rope_cos;  // [n_pos][d/2] or null
  const float* rope_sin;
  const int32_t* lens;    // [B] current lengths
  int32_t* lens_out;      // [B] lengths after the append, or null
  uint16_t* v_tail;       // [B][Hkv][32][d] raw values of each open value block (in/out)
  uint8_t* q_codes;
  uint8_t* q_scales;
  uint8_t* k_codes;       // cache, row layout with capacity cap
  uint8_t* k_scales;
  uint8_t* v_codes;       // cache, column layout with capacity cap
  uint8_t* v_scales;
  int B, Hq, Hkv, n_new, d, cap;
  int n_pos, q_pos0, k_pos0;
  uint32_t q_bias, k_bias, v_bias;  // block-scale rule of each output (kScaleBias*)
  int64_t blocks_q, blocks_k, wg_q, wg_k, items_v;  // filled by the launcher
};

hipError_t launch_kv_append(AppendArgs a, bool bf16, hipStream_t stream);

struct CalibrateArgs {
  const uint16_t* q;     // [B][Hq][S][d]
  const uint16_t* k;     // [B][Hkv][S][d]
  float* smooth;         // [Hkv][d]
  uint32_t* workspace;   // 2 * Hkv * d words: max|K| then max|Q| bit patterns
  const float* rope_cos; // rotate-half RoPE tables [n_pos][d/2], or null
  const float* rope_sin;
  int q_pos0, k_pos0;
  int B, Hq, Hkv, S, d;
  double alpha;
};

hipError_t launch_smooth_calibrate(const CalibrateArgs& a, bool bf16, hipStream_t stream);

// Attention problem after validation; pointers are device pointers.
struct AttnArgs {
  const uint8_t* q_codes;
  const uint8_t* q_scales;
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  void* out;
  float* lse;
  const uint16_t* q_raw;   // prefill: bf16 / fp16 Q quantised in the kernel (q_codes unused), or null
  const float* smooth;     // with q_raw: Smooth-QK factors [Hkv][d], or null (s = 1)
  int q_raw_bf16;          // with q_raw: 1 = bf16, 0 = fp16
  const int32_t* kv_lens;  // decode only, may be null
  float* partials;         // decode workspace
  int B, Hq, Hkv, Sq, Sk, d, cap;
  int causal;
  int out_fp16;
  float sm_log2;           // sm_scale * log2(e)
  float sm_scale;
  int chunk;               // decode: tokens per piece given by the caller, 0 = balanced
  int dec_waves;           // decode: waves of the persistent grid
  float tau;               // lazy-rescale threshold, log2 units (0 = every increase)
  int direct_l;            // 1: l = sum of the fp32 P (vector ALU), 0: P-Reordering
  uint32_t p_bias;         // block-scale rule of P_hat (kScaleBias*)
  uint32_t q_bias;         // with q_raw: block-scale rule of the in-kernel Q quantisation
};

// Key tile width of the online-softmax frame for a head dim.
int attn_block_n(int d);
// Waves of the persistent decode grid for a head dim.
int attn_decode_waves(int d);

// Key tiles per decode piece: the caller's chunk (tokens, a multiple of the
// 64-key tile), else an even share of the total over the grid's waves.
__host__ __device__ inline int decode_piece_tiles(int chunk, int waves, int total_tiles) {
  if (chunk > 0) return chunk / 64;
  const int p = (total_tiles + waves - 1) / waves;
  return p > 1 ? p : 1;
}

hipError_t launch_attn_prefill_mxfp4(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_decode_mxfp4(const AttnArgs& a, hipStream_t stream);

// Device scratch of the allocation-free entry point: bytes per device, and its
// device address on the current device (looked up on the first call there).
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
hipError_t static_scratch(void** ptr);

struct Bf16AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* lse;
  int B, Hq, Hkv, Sq, Sk, d, cap;
  int causal;
  float sm_log2;
  float tau;
};

hipError_t launch_attn_prefill_bf16(const Bf16AttnArgs& a, hipStream_t stream);

}  // namespace hifa4
