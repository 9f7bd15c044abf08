// probes.hip -- diagnostic kernels that pin down gfx950 instruction behaviour
// the attention kernels rely on: the operand / scale / accumulator lane
// layouts of the scaled-FP4 and bf16 MFMAs, the rounding of the packed FP4
// convert, the lane placement of memory -> LDS buffer loads, the issue
// rates of v_exp_f32 and the FP4 MFMA, and the HBM read rate of a plain
// streaming kernel.
//
// Built into its own library (libhifa4_probes.so); the tests call it to check
// those facts against independent host-side expectations.  Every kernel reads
// and writes exactly the buffers sized by its arguments.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "hifa4_probes.h"

namespace hifa4 {
namespace {

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, size_t n16,
                                                         uint32_t* __restrict__ out) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

template <int kOpsel>
__global__ __launch_bounds__(64) void mfma_fp4_32_kernel(const uint4* a, const uint4* b,
                                                         const uint32_t* sa, const uint32_t* sb,
                                                         float* d) {
  const int w = blockIdx.x, l = threadIdx.x;
  v16f c = {};
  v8i A = {(int)a[w * 64 + l].x, (int)a[w * 64 + l].y, (int)a[w * 64 + l].z, (int)a[w * 64 + l].w,
           0, 0, 0, 0};
  v8i B = {(int)b[w * 64 + l].x, (int)b[w * 64 + l].y, (int)b[w * 64 + l].z, (int)b[w * 64 + l].w,
           0, 0, 0, 0};
  c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c, kFmtFp4, kFmtFp4, kOpsel,
                                                      (int)sa[w * 64 + l], kOpsel,
                                                      (int)sb[w * 64 + l]);
#pragma unroll
  for (int r = 0; r < 16; r++) d[(w * 64 + l) * 16 + r] = c[r];
}

template <int kOpsel>
__global__ __launch_bounds__(64) void mfma_fp4_16_kernel(const uint4* a, const uint4* b,
                                                         const uint32_t* sa, const uint32_t* sb,
                                                         float* d) {
  const int w = blockIdx.x, l = threadIdx.x;
  v4f c = {};
  v8i A = {(int)a[w * 64 + l].x, (int)a[w * 64 + l].y, (int)a[w * 64 + l].z, (int)a[w * 64 + l].w,
           0, 0, 0, 0};
  v8i B = {(int)b[w * 64 + l].x, (int)b[w * 64 + l].y, (int)b[w * 64 + l].z, (int)b[w * 64 + l].w,
           0, 0, 0, 0};
  c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, kFmtFp4, kFmtFp4, kOpsel,
                                                       (int)sa[w * 64 + l], kOpsel,
                                                       (int)sb[w * 64 + l]);
#pragma unroll
  for (int r = 0; r < 4; r++) d[(w * 64 + l) * 4 + r] = c[r];
}

__global__ __launch_bounds__(64) void mfma_bf16_32_kernel(const uint4* a, const uint4* b,
                                                          float* d) {
  const int w = blockIdx.x, l = threadIdx.x;
  uint4 x = a[w * 64 + l], y = b[w * 64 + l];
  v8s A, B;
  __builtin_memcpy(&A, &x, 16);
  __builtin_memcpy(&B, &y, 16);
  v16f c = {};
  c = mfma_bf16_32x32x16(A, B, c);
#pragma unroll
  for (int r = 0; r < 16; r++) d[(w * 64 + l) * 16 + r] = c[r];
}

__global__ __launch_bounds__(64) void half_swap_kernel(const float* x, float* out) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  const float v = x[i];
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  out[2 * i] = __uint_as_float(r[0]);
  out[2 * i + 1] = __uint_as_float(r[1]);
}

template <int kSel>
__global__ void cvt_fp4_kernel(const float2* x, const float* scale, uint32_t* out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[i].x, x[i].y, scale[i], kSel);
  out[i] = r;
}

__global__ void exp2_rate_kernel(float* out, int iters) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; j++) x[j] = 0.001f * (threadIdx.x + j);
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int j = 0; j < 8; j++) x[j] = __builtin_amdgcn_exp2f(-x[j]);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; j++) s += x[j];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void mfma_rate_kernel(float* out, int iters) {
  const int l = threadIdx.x;
  uint4 a = make_uint4(0x22222222u ^ l, 0x12345678u, 0x0u, 0x76543210u);
  uint4 b = make_uint4(0x11111111u, 0x22222222u ^ l, 0x33333333u, 0x0u);
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  int s = 127 + (l & 1);
  for (int it = 0; it < iters; it++) {
    c0 = mfma_fp4_32x32x64(a, b, c0, s, s);
    c1 = mfma_fp4_32x32x64(b, a, c1, s, s);
    c2 = mfma_fp4_32x32x64(a, a, c2, s, s);
    c3 = mfma_fp4_32x32x64(b, b, c3, s, s);
  }
  float t = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; r++) t += c0[r] + c1[r] + c2[r] + c3[r];
  out[blockIdx.x * blockDim.x + l] = t;
}

// The same for the 16 x 16 x 128 FP4 MFMA (half the multiply-adds of the
// 32 x 32 x 64 form per instruction, a quarter of its accumulator): eight
// independent chains per wave.
__global__ __launch_bounds__(256) void mfma16_rate_kernel(float* out, int iters) {
  const int l = threadIdx.x;
  v8i A = {(int)(0x22222222u ^ l), 0x12345678, 0, 0x76543210, 0, 0, 0, 0};
  v8i B = {0x11111111, (int)(0x22222222u ^ l), 0x33333333, 0, 0, 0, 0, 0};
  v4f c[8];
#pragma unroll
  for (int j = 0; j < 8; j++) c[j] = v4f{};
  int s = 127 + (l & 1);
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int j = 0; j < 8; j++)
      c[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(j & 1 ? B : A, j & 2 ? A : B, c[j],
                                                              kFmtFp4, kFmtFp4, 0, s, 0, s);
  }
  float t = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; j++) t += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  out[blockIdx.x * blockDim.x + l] = t;
}

// Issue cost of vector instructions, two waves per SIMD, 8 independent chains
// per wave, 32 instructions per wave and iteration (modes as in the header).
template <int MODE>
__global__ __launch_bounds__(512) void valu_rate_kernel(float* out, int iters) {
  const int w = threadIdx.x >> 6;
  float x[8], y[8];
  uint32_t pk[8];
#pragma unroll
  for (int j = 0; j < 8; j++) {
    x[j] = 0.001f * (threadIdx.x + j) - 0.5f;
    y[j] = 0.3f + 0.01f * j;
    pk[j] = 0;
  }
  auto fma1 = [](float v) { return __builtin_fmaf(v, 0.999f, -0.001f); };
  auto cvt1 = [](uint32_t p, float a, float b) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, a, b, 1.0f, 0);
  };
  if constexpr (MODE == 6) {
    if (w < 4) {
      for (int it = 0; it < iters; it++)
#pragma unroll
        for (int r = 0; r < 32; r++) x[r & 7] = __builtin_amdgcn_exp2f(x[r & 7]);
    } else {
      for (int it = 0; it < iters; it++)
#pragma unroll
        for (int r = 0; r < 32; r++) x[r & 7] = fma1(x[r & 7]);
    }
  } else {
    for (int it = 0; it < iters; it++) {
#pragma unroll
      for (int r = 0; r < 32; r++) {
        const int j = r & 7;
        const bool odd = r & 1;
        if constexpr (MODE == 0) x[j] = fma1(x[j]);
        if constexpr (MODE == 1) x[j] = __builtin_amdgcn_exp2f(x[j]);
        if constexpr (MODE == 2) x[j] = odd ? __builtin_amdgcn_exp2f(x[j]) : fma1(x[j]);
        if constexpr (MODE == 3) {
          if (odd) pk[j] = cvt1(pk[j], x[j], y[j]);
          else x[j] = fma1(x[j]);
        }
        if constexpr (MODE == 4)
          x[j] = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[j], y[j]),
                                               x[(j + 1) & 7]);
        if constexpr (MODE == 5) {
          if (odd) pk[j] = cvt1(pk[j], x[j], y[j]);
          else x[j] = __builtin_amdgcn_exp2f(x[j]);
        }
      }
    }
  }
  float t = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; j++) t += x[j] + (float)pk[j];
  out[blockIdx.x * blockDim.x + threadIdx.x] = t;
}

// Co-execution of the matrix core and the vector ALU: 512-thread blocks (two
// waves per SIMD), per iteration 16 FP4 32x32x64 MFMAs (four independent
// chains) and 32 exp2(fma) pairs (eight independent chains).  mode 0: MFMAs
// only; 1: vector work only; 2: both, interleaved in every wave; 3: waves 0-3
// (one per SIMD) the MFMAs, waves 4-7 the vector work, so each SIMD holds one
// wave of each kind.
__global__ __launch_bounds__(512) void coexec_kernel(float* out, int mode, int iters) {
  const int l = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const uint4 a = make_uint4(0x22222222u ^ l, 0x12345678u, 0x0u, 0x76543210u);
  const uint4 b = make_uint4(0x11111111u, 0x22222222u ^ l, 0x33333333u, 0x0u);
  v16f c[4];
#pragma unroll
  for (int j = 0; j < 4; j++) c[j] = v16f{};
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; j++) x[j] = 0.001f * (threadIdx.x + j);
  const int s = 127 + (l & 1);
  const bool do_m = mode == 0 || mode == 2 || (mode == 3 && w < 4);
  const bool do_v = mode == 1 || mode == 2 || (mode == 3 && w >= 4);
  if (mode == 2) {
    for (int it = 0; it < iters; it++) {
#pragma unroll
      for (int i = 0; i < 16; i++) c[i % 4] = mfma_fp4_32x32x64(i & 1 ? a : b, i & 2 ? b : a, c[i % 4], s, s);
#pragma unroll
      for (int j = 0; j < 32; j++)
        x[j % 8] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j % 8], 0.5f, -0.25f));
#pragma unroll
      for (int i = 0; i < 16; i++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
    }
  } else {
    if (do_m)
      for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int i = 0; i < 16; i++)
          c[i % 4] = mfma_fp4_32x32x64(i & 1 ? a : b, i & 2 ? b : a, c[i % 4], s, s);
      }
    if (do_v)
      for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int j = 0; j < 32; j++)
          x[j % 8] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j % 8], 0.5f, -0.25f));
      }
  }
  float t = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int r = 0; r < 16; r++) t += c[j][r];
#pragma unroll
  for (int j = 0; j < 8; j++) t += x[j];
  out[blockIdx.x * 512 + threadIdx.x] = t;
}

// The gfx950 LDS transpose read of 16-bit elements (ds_read_b64_tr_b16):
// LDS holds element i = i (as 16 bits) over 4096 elements; lane l reads at
// element offset addr[l] (a multiple of 4) and returns 4 elements to
// out[4l .. 4l+3].
typedef short v4s_probe __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(64) void lds_read_tr16_kernel(const int* addr, short* out) {
  __shared__ __attribute__((aligned(16))) short lds[4096];
  for (int i = threadIdx.x; i < 4096; i += 64) lds[i] = (short)i;
  __syncthreads();
  typedef __attribute__((address_space(3))) v4s_probe* lp;
  const lp p = (lp)((__attribute__((address_space(3))) short*)lds + addr[threadIdx.x]);
  const v4s_probe r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
  for (int e = 0; e < 4; e++) out[threadIdx.x * 4 + e] = r[e];
}

// Memory -> LDS buffer loads (the LDS-destination form): one wave loads
// `size`-byte elements, lane i from source byte offset size*i, with M0 = 64;
// the LDS window is pre-filled with 0xEE and copied out afterwards, so the
// host sees where each lane's bytes landed.  The window (1 KiB + 64) covers
// every placement the sizes allow.
template <int kSize>
__global__ __launch_bounds__(64) void lds_dma_kernel(const uint8_t* src, uint8_t* out) {
  __shared__ __attribute__((aligned(16))) uint8_t win[64 + 16 * 64];
  const int l = threadIdx.x;
  for (int i = l; i < (int)sizeof(win); i += 64) win[i] = 0xEE;
  __syncthreads();
  typedef int v4i __attribute__((ext_vector_type(4)));
  const uint64_t p = reinterpret_cast<uint64_t>(src);
  v4i d;
  d[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  d[1] = __builtin_amdgcn_readfirstlane((int)((p >> 32) & 0xFFFFu));
  d[2] = 16 * 64;
  d[3] = 0x00020000;
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)reinterpret_cast<uintptr_t>(win + 64));
  const uint32_t off = (uint32_t)(kSize * l);
  if constexpr (kSize == 1)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_ubyte %1, %2, 0 offen lds" ::"s"(m0), "v"(off), "s"(d) : "memory");
  else if constexpr (kSize == 2)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_ushort %1, %2, 0 offen lds" ::"s"(m0), "v"(off), "s"(d) : "memory");
  else if constexpr (kSize == 4)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(m0), "v"(off), "s"(d) : "memory");
  else
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(off), "s"(d) : "memory");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int i = l; i < (int)sizeof(win); i += 64) out[i] = win[i];
}


// Raw buffer range check: one wave loads dword i from voffset 4i with the
// given soffset and num_records (src must hold soffset + 256 bytes); lanes
// whose load is out of range read 0.  The first 64 outputs come from a
// register load, the next 64 from the memory -> LDS form.
__global__ __launch_bounds__(64) void buffer_range_kernel(const uint32_t* src, uint32_t* out,
                                                          int soffset, int num_records) {
  __shared__ __attribute__((aligned(16))) uint32_t win[64];
  const int l = threadIdx.x;
  win[l] = 0xEEEEEEEEu;
  __syncthreads();
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, num_records, 0x00020000);
  out[l] = __builtin_amdgcn_raw_buffer_load_b32(r, (uint32_t)(4 * l), soffset, 0);
  typedef int v4i __attribute__((ext_vector_type(4)));
  const uint64_t p = reinterpret_cast<uint64_t>(src);
  v4i d;
  d[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  d[1] = __builtin_amdgcn_readfirstlane((int)((p >> 32) & 0xFFFFu));
  d[2] = __builtin_amdgcn_readfirstlane(num_records);
  d[3] = 0x00020000;
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)reinterpret_cast<uintptr_t>(win));
  const int so = __builtin_amdgcn_readfirstlane(soffset);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               ::"s"(m0), "v"((uint32_t)(4 * l)), "s"(d), "s"(so) : "memory");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  out[64 + l] = win[l];
}

int status(hipError_t e) { return e == hipSuccess ? 0 : -(int)e; }

}  // namespace
}  // namespace hifa4

using namespace hifa4;

extern "C" {

int probe_mfma_fp4_32x32x64(const uint32_t* a, const uint32_t* b, const uint32_t* sa,
                            const uint32_t* sb, float* d, int n_waves, int opsel, void* stream) {
  if (n_waves <= 0 || opsel < 0 || opsel > 3) return -1;
  auto s = (hipStream_t)stream;
  auto A = reinterpret_cast<const uint4*>(a);
  auto B = reinterpret_cast<const uint4*>(b);
  switch (opsel) {
    case 0: hipLaunchKernelGGL(mfma_fp4_32_kernel<0>, dim3(n_waves), dim3(64), 0, s, A, B, sa, sb, d); break;
    case 1: hipLaunchKernelGGL(mfma_fp4_32_kernel<1>, dim3(n_waves), dim3(64), 0, s, A, B, sa, sb, d); break;
    case 2: hipLaunchKernelGGL(mfma_fp4_32_kernel<2>, dim3(n_waves), dim3(64), 0, s, A, B, sa, sb, d); break;
    default: hipLaunchKernelGGL(mfma_fp4_32_kernel<3>, dim3(n_waves), dim3(64), 0, s, A, B, sa, sb, d); break;
  }
  return status(hipGetLastError());
}

int probe_mfma_fp4_16x16x128(const uint32_t* a, const uint32_t* b, const uint32_t* sa,
                             const uint32_t* sb, float* d, int n_waves, int opsel, void* stream) {
  if (n_waves <= 0 || opsel < 0 || opsel > 3) return -1;
  auto s = (hipStream_t)stream;
  auto A = reinterpret_cast<const uint4*>(a);
  auto B = reinterpret_cast<const uint4*>(b);
  switch (opsel) {
    case 0: hipLaunchKernelGGL(mfma_fp4_16_kernel<0>, dim3(n_waves), dim3(64), 0, s, A, B, sa, sb, d); break;
    case 1: hipLaunchKernelGGL(mfma_fp4_16_kernel<1>, dim3(n_waves), dim3(64), 0, s, A, B, sa, sb, d); break;
    case 2: hipLaunchKernelGGL(mfma_fp4_16_kernel<2>, dim3(n_waves), dim3(64), 0, s, A, B, sa, sb, d); break;
    default: hipLaunchKernelGGL(mfma_fp4_16_kernel<3>, dim3(n_waves), dim3(64), 0, s, A, B, sa, sb, d); break;
  }
  return status(hipGetLastError());
}

int probe_mfma_bf16_32x32x16(const uint16_t* a, const uint16_t* b, float* d, int n_waves,
                             void* stream) {
  if (n_waves <= 0) return -1;
  hipLaunchKernelGGL(mfma_bf16_32_kernel, dim3(n_waves), dim3(64), 0, (hipStream_t)stream,
                     reinterpret_cast<const uint4*>(a), reinterpret_cast<const uint4*>(b), d);
  return status(hipGetLastError());
}

int probe_cvt_pk_fp4(const float* x, const float* scale, uint32_t* out, int n, int sel,
                     void* stream) {
  if (n <= 0 || sel < 0 || sel > 3) return -1;
  auto s = (hipStream_t)stream;
  auto X = reinterpret_cast<const float2*>(x);
  dim3 g((n + 255) / 256), t(256);
  switch (sel) {
    case 0: hipLaunchKernelGGL(cvt_fp4_kernel<0>, g, t, 0, s, X, scale, out, n); break;
    case 1: hipLaunchKernelGGL(cvt_fp4_kernel<1>, g, t, 0, s, X, scale, out, n); break;
    case 2: hipLaunchKernelGGL(cvt_fp4_kernel<2>, g, t, 0, s, X, scale, out, n); break;
    default: hipLaunchKernelGGL(cvt_fp4_kernel<3>, g, t, 0, s, X, scale, out, n); break;
  }
  return status(hipGetLastError());
}

int probe_half_swap(const float* x, float* out, int n_waves, void* stream) {
  if (n_waves <= 0) return -1;
  hipLaunchKernelGGL(half_swap_kernel, dim3(n_waves), dim3(64), 0, (hipStream_t)stream, x, out);
  return status(hipGetLastError());
}

int probe_stream_read(const void* src, size_t bytes, uint32_t* out, int n_blocks, void* stream) {
  if (!src || !out || n_blocks <= 0 || (bytes & 15)) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(n_blocks), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const uint4*>(src), bytes / 16, out);
  return status(hipGetLastError());
}

int probe_exp2_rate(float* out, int n_blocks, int iters, void* stream) {
  if (n_blocks <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(exp2_rate_kernel, dim3(n_blocks), dim3(256), 0, (hipStream_t)stream, out,
                     iters);
  return status(hipGetLastError());
}

int probe_mfma_rate(float* out, int n_blocks, int iters, void* stream) {
  if (n_blocks <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(n_blocks), dim3(256), 0, (hipStream_t)stream, out,
                     iters);
  return status(hipGetLastError());
}

int probe_mfma16_rate(float* out, int n_blocks, int iters, void* stream) {
  if (n_blocks <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma16_rate_kernel, dim3(n_blocks), dim3(256), 0, (hipStream_t)stream, out,
                     iters);
  return status(hipGetLastError());
}

int probe_coexec(float* out, int mode, int n_blocks, int iters, void* stream) {
  if (n_blocks <= 0 || iters <= 0 || mode < 0 || mode > 3) return -1;
  hipLaunchKernelGGL(coexec_kernel, dim3(n_blocks), dim3(512), 0, (hipStream_t)stream, out, mode,
                     iters);
  return status(hipGetLastError());
}

int probe_valu_rate(float* out, int mode, int n_blocks, int iters, void* stream) {
  if (n_blocks <= 0 || iters <= 0) return -1;
  const dim3 g(n_blocks), b(512);
  hipStream_t st = (hipStream_t)stream;
  switch (mode) {
    case 0: hipLaunchKernelGGL(valu_rate_kernel<0>, g, b, 0, st, out, iters); break;
    case 1: hipLaunchKernelGGL(valu_rate_kernel<1>, g, b, 0, st, out, iters); break;
    case 2: hipLaunchKernelGGL(valu_rate_kernel<2>, g, b, 0, st, out, iters); break;
    case 3: hipLaunchKernelGGL(valu_rate_kernel<3>, g, b, 0, st, out, iters); break;
    case 4: hipLaunchKernelGGL(valu_rate_kernel<4>, g, b, 0, st, out, iters); break;
    case 5: hipLaunchKernelGGL(valu_rate_kernel<5>, g, b, 0, st, out, iters); break;
    case 6: hipLaunchKernelGGL(valu_rate_kernel<6>, g, b, 0, st, out, iters); break;
    default: return -1;
  }
  return status(hipGetLastError());
}

int probe_lds_read_tr16(const int* addr, short* out, void* stream) {
  hipLaunchKernelGGL(lds_read_tr16_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, addr, out);
  return status(hipGetLastError());
}

int probe_lds_dma(const uint8_t* src, uint8_t* out, int size, void* stream) {
  auto s = (hipStream_t)stream;
  switch (size) {
    case 1: hipLaunchKernelGGL(lds_dma_kernel<1>, dim3(1), dim3(64), 0, s, src, out); break;
    case 2: hipLaunchKernelGGL(lds_dma_kernel<2>, dim3(1), dim3(64), 0, s, src, out); break;
    case 4: hipLaunchKernelGGL(lds_dma_kernel<4>, dim3(1), dim3(64), 0, s, src, out); break;
    case 16: hipLaunchKernelGGL(lds_dma_kernel<16>, dim3(1), dim3(64), 0, s, src, out); break;
    default: return -1;
  }
  return status(hipGetLastError());
}

int probe_buffer_range(const uint32_t* src, uint32_t* out, int soffset, int num_records,
                       void* stream) {
  if (soffset < 0 || (soffset & 3) || num_records < 0) return -1;
  hipLaunchKernelGGL(buffer_range_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, src, out,
                     soffset, num_records);
  return status(hipGetLastError());
}

}  // extern "C"
