// stub_launch.cpp -- host-only stand-ins for the kernel launchers behind the C
// ABI, so that api.cpp can be built with the host compiler under
// AddressSanitizer and driven without a GPU.  Each launcher only counts its
// calls; nothing here touches device memory.
#include <hip/hip_runtime.h>

#include "launch.hpp"

int g_launches = 0;

extern "C" const char* hipGetErrorString(hipError_t) { return "stub HIP error"; }

namespace hifa4 {

hipError_t launch_quantize_qkv(QuantizeArgs, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_kv_append(AppendArgs, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_smooth_calibrate(const CalibrateArgs&, bool, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_attn_prefill_mxfp4(const AttnArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_attn_decode_mxfp4(const AttnArgs& a, hipStream_t) {
  ++g_launches;
  // the decode path must have been given workspace for its partials
  return a.partials ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_attn_prefill_bf16(const Bf16AttnArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
int attn_block_n(int) { return 64; }
int attn_decode_waves(int d) { return d == 256 ? 1024 : 2048; }
hipError_t static_scratch(void** p) {
  *p = reinterpret_cast<void*>(uintptr_t(0x7F000000));
  return hipSuccess;
}

}  // namespace hifa4
