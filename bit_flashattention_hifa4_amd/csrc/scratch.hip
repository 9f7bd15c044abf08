// scratch.hip -- device-resident scratch of the attention entry point that
// allocates nothing (hifa4_attn_fwd_noalloc).
//
// The split-K decode keeps one partial row (m, l, acc) per run in scratch
// memory.  hifa4_attn_fwd takes that memory from the caller; callers that
// cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc) get it from the file-scope array below
// instead.  Every GPU the library runs on holds its own copy of the array
// for the life of the process, at its own device address.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is ever passed to a kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

static __device__ __align__(256) unsigned char scratch[hifa4::kStaticScratchBytes];

namespace hifa4 {

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace hifa4
