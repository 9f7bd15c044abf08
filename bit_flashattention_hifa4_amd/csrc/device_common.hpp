// device_common.hpp -- gfx950 device helpers shared by the library's kernels.
//
// Scaled-FP4 MFMA wrappers, E8M0 helpers and small conversions.  Only the HIP
// library includes this file.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hifa4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));

// Operand-format selector of the f8f6f4 MFMA family for FP4 E2M1.
constexpr int kFmtFp4 = 4;

// D = A * B + C on 32 x 32 x 64 FP4 tiles with E8M0 block scales.
// Lane l supplies row (l % 32) of A / column (l % 32) of B, 32 consecutive
// K elements (block l / 32) packed in 16 bytes, plus that block's scale in
// byte 0 of sa / sb.  The accumulator holds D[m][n] for n = l % 32,
// m = 8 * (r / 4) + 4 * (l / 32) + r % 4 in register r.
__device__ __forceinline__ v16f mfma_fp4_32x32x64(const uint4& a, const uint4& b, const v16f& c,
                                                  int sa, int sb) {
  v8i A = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  v8i B = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c, kFmtFp4, kFmtFp4, 0, sa, 0, sb);
}

// bf16 MFMA 32 x 32 x 16: lane l supplies row / column (l % 32) and K
// elements 8 * (l / 32) .. + 7; accumulator layout as above.
__device__ __forceinline__ v16f mfma_bf16_32x32x16(const v8s& a, const v8s& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// E8M0 byte of a block's shared exponent for a non-negative finite fp32 amax:
// with bias 0 the OCP MX exponent floor(log2(amax)) - 2, i.e. the fp32
// exponent field minus 2, floored at 0 (zero and tiny blocks get exponent
// -127).  A bias of 2^22 - 1 (the no-clip rule) carries into the exponent
// field exactly when the mantissa exceeds 1.5, i.e. when amax > 6 * 2^X for
// that OCP exponent X, so the exponent rises by one precisely where an element
// would otherwise saturate at 6.
__device__ __forceinline__ uint32_t e8m0_from_amax(float amax, uint32_t bias) {
  int ef = (int)((__float_as_uint(amax) + bias) >> 23);
  return (uint32_t)max(ef - 2, 0);
}

// fp32 value 2^(byte - 127) of an E8M0 byte in [1, 254]; byte 0 maps to
// 2^-127 as a denormal.
__device__ __forceinline__ float e8m0_to_float(uint32_t byte) {
  return byte ? __uint_as_float(byte << 23) : __uint_as_float(0x00400000u);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t float_to_half_bits(float f) {
  return (uint32_t)__half_as_ushort(__float2half_rn(f));
}

// Exact fp32 value of a bf16 (kBf16) or fp16 element.
template <bool kBf16>
__device__ __forceinline__ float elem(uint32_t bits16) {
  if constexpr (kBf16) {
    return bf16_bits_to_float(bits16);
  } else {
    return __half2float(__ushort_as_half((unsigned short)bits16));
  }
}

// 8 elements -> 4 E2M1 code bytes (element 2i in the low nibble of byte i):
// the gfx950 packed convert divides by the power-of-two scale, rounds to
// nearest even and saturates at +-6.
__device__ __forceinline__ uint32_t encode8(const float (&v)[8], float scale) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], scale, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], scale, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], scale, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], scale, 3);
  return w;
}

}  // namespace hifa4
