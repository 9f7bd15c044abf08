// lds_dma.hpp -- memory -> LDS buffer loads (the LDS-destination form of
// buffer_load) and the buffer descriptors they take.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hifa4 {

typedef int v4i __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (stride 0) over `bytes` bytes from `base`: loads at
// or past `bytes` return zeros.  Word 3 is the gfx9-family default format.
__device__ __forceinline__ v4i buffer_desc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  r[1] = __builtin_amdgcn_readfirstlane((int)((p >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)reinterpret_cast<uintptr_t>(p));
}

// Memory -> LDS, 16 / 4 / 2 bytes per lane, from buffer offset soff + off:
// lane i writes LDS bytes [lds + size*i, lds + size*(i+1)); the 2-byte form
// writes a zero-extended dword at lds + 4i.  The range check counts soff, so
// one descriptor over a head's valid keys serves every tile.  (Placement and
// range behaviour are pinned by the LDS-load probes.)
// M0 = lds + LDS_IMM (the per-stage part of the address as a constant).
// The asm sets M0 with s_mov, which leaves SCC alone: the compiler does not
// model an SCC clobber and may keep a pending s_cselect condition in SCC
// across the statement.  M0 holds nothing else in these kernels.
template <int LDS_IMM>
__device__ __forceinline__ void load_lds16(v4i desc, uint32_t off, int soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds + LDS_IMM), "v"(off), "s"(desc), "s"(soff) : "memory");
}
template <int LDS_IMM>
__device__ __forceinline__ void load_lds4(v4i desc, uint32_t off, int soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds + LDS_IMM), "v"(off), "s"(desc), "s"(soff) : "memory");
}
template <int LDS_IMM>
__device__ __forceinline__ void load_lds2(v4i desc, uint32_t off, int soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_ushort %1, %2, %3 offen lds"
               :: "s"(lds + LDS_IMM), "v"(off), "s"(desc), "s"(soff) : "memory");
}

// vmcnt(n) with the other counters left alone (gfx9 encoding; n < 16).
#define HIFA4_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | (n))

}  // namespace hifa4
