// abi_driver.cpp -- drives every entry point of include/hifa4.h through its
// validation paths and a valid call each, with the launchers stubbed out
// (stub_launch.cpp), under AddressSanitizer / UndefinedBehaviorSanitizer.
// Pointers are fake, 16-byte aligned device addresses that are never
// dereferenced.  Checks: the documented status for each case; nothing
// launched when a call fails; the error text set on failure and cleared on
// success.  Exit status 0 when every check passes.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "hifa4.h"

extern int g_launches;

static int g_fail = 0;

#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                         \
    }                                                                   \
  } while (0)

static uint8_t* P(uintptr_t a) { return reinterpret_cast<uint8_t*>(a); }

// A call that must fail with `want` and launch nothing.
#define EXPECT_FAIL(want, call)                                         \
  do {                                                                  \
    const int before = g_launches;                                      \
    const hifa4_status st = (call);                                     \
    CHECK(st == (want));                                                \
    CHECK(g_launches == before);                                        \
    CHECK(std::strlen(hifa4_last_error()) > 0);                         \
  } while (0)

// A call that must succeed and launch `n` kernels.
#define EXPECT_OK(n, call)                                              \
  do {                                                                  \
    const int before = g_launches;                                      \
    const hifa4_status st = (call);                                     \
    CHECK(st == HIFA4_OK);                                              \
    CHECK(g_launches == before + (n));                                  \
    CHECK(std::strlen(hifa4_last_error()) == 0);                        \
  } while (0)

static hifa4_attn_params params(int Sq) {
  hifa4_attn_params p;
  std::memset(&p, 0, sizeof p);
  p.B = 2; p.Hq = 8; p.Hkv = 2; p.Sq = Sq; p.Sk = 300; p.d = 128; p.causal = 1;
  p.kv_stride = 320;
  return p;
}

static hifa4_mx_tensor mx(uintptr_t base) { return hifa4_mx_tensor{P(base), P(base + 0x1000000), 0}; }

int main() {
  const hifa4_mx_tensor q = mx(0x10000000), k = mx(0x20000000), v = mx(0x30000000);
  void* out = P(0x40000000);
  float* lse = reinterpret_cast<float*>(0x50000000);
  void* ws = P(0x60000000);

  // ---- attention: parameters
  hifa4_attn_params p = params(128);
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT,
              hifa4_attn_fwd(nullptr, q, k, v, out, HIFA4_BF16, lse, nullptr, 0, nullptr));
  p.d = 96;
  EXPECT_FAIL(HIFA4_ERR_UNSUPPORTED, hifa4_attn_fwd(&p, q, k, v, out, HIFA4_BF16, lse, nullptr, 0, nullptr));
  p = params(128); p.Hkv = 3;
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_attn_fwd(&p, q, k, v, out, HIFA4_BF16, lse, nullptr, 0, nullptr));
  p = params(128); p.rescale_threshold = 65.0f;
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_attn_fwd(&p, q, k, v, out, HIFA4_BF16, lse, nullptr, 0, nullptr));
  p = params(128); p.rescale_threshold = NAN;
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_attn_fwd(&p, q, k, v, out, HIFA4_BF16, lse, nullptr, 0, nullptr));
  p = params(128); p.kv_stride = 100;
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_attn_fwd(&p, q, k, v, out, HIFA4_BF16, lse, nullptr, 0, nullptr));
  p = params(128); p.Sk = 1 << 24; p.kv_stride = 0; p.d = 256;
  EXPECT_FAIL(HIFA4_ERR_UNSUPPORTED, hifa4_attn_fwd(&p, q, k, v, out, HIFA4_BF16, lse, nullptr, 0, nullptr));
  p = params(128); p.decode_chunk = 64;
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_attn_fwd(&p, q, k, v, out, HIFA4_BF16, lse, nullptr, 0, nullptr));
  p = params(128); p.normaliser = 2;
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_attn_fwd(&p, q, k, v, out, HIFA4_BF16, lse, nullptr, 0, nullptr));
  p = params(128); p.scale_rule = 9;
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_attn_fwd(&p, q, k, v, out, HIFA4_BF16, lse, nullptr, 0, nullptr));
  // ---- attention: pointers
  p = params(128);
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_attn_fwd(&p, q, k, v, nullptr, HIFA4_BF16, lse, nullptr, 0, nullptr));
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_attn_fwd(&p, q, k, v, P(0x40000008), HIFA4_BF16, lse, nullptr, 0, nullptr));
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_attn_fwd(&p, q, k, v, P(0x10000000), HIFA4_BF16, lse, nullptr, 0, nullptr));
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_attn_fwd(&p, q, k, v, out, (hifa4_dtype)5, lse, nullptr, 0, nullptr));
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_attn_fwd(&p, q, k, v, out, HIFA4_BF16, reinterpret_cast<float*>(0x40000000), nullptr, 0, nullptr));
  // ---- attention: valid prefill, empty problem, decode with and without workspace
  EXPECT_OK(1, hifa4_attn_fwd(&p, q, k, v, out, HIFA4_BF16, lse, nullptr, 0, nullptr));
  EXPECT_OK(1, hifa4_attn_fwd(&p, q, k, v, out, HIFA4_FP16, nullptr, nullptr, 0, nullptr));
  p.B = 0;
  EXPECT_OK(0, hifa4_attn_fwd(&p, q, k, v, out, HIFA4_BF16, lse, nullptr, 0, nullptr));
  hifa4_attn_params dp = params(1);
  const size_t need = hifa4_attn_workspace_size(&dp);
  CHECK(need > 0);
  EXPECT_FAIL(HIFA4_ERR_WORKSPACE_TOO_SMALL, hifa4_attn_fwd(&dp, q, k, v, out, HIFA4_BF16, lse, ws, need - 1, nullptr));
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_attn_fwd(&dp, q, k, v, out, HIFA4_BF16, lse, nullptr, need, nullptr));
  EXPECT_OK(1, hifa4_attn_fwd(&dp, q, k, v, out, HIFA4_BF16, lse, ws, need, nullptr));
  dp.decode_chunk = 192;
  EXPECT_OK(1, hifa4_attn_fwd(&dp, q, k, v, out, HIFA4_BF16, lse, ws, hifa4_attn_workspace_size(&dp), nullptr));
  // ---- schedule queries
  int32_t bn = 0, ch = -1;
  CHECK(hifa4_attn_schedule(&dp, &bn, &ch) == HIFA4_OK && bn == 64 && ch == 192);
  CHECK(hifa4_attn_decode_piece_tiles(&dp, 100) == 3);
  p = params(128);
  CHECK(hifa4_attn_decode_piece_tiles(&p, 100) == 0);
  p.d = 7;
  CHECK(hifa4_attn_workspace_size(&p) == 0);
  // ---- Q from activations
  p = params(128);
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_attn_fwd_qraw(&p, nullptr, HIFA4_BF16, nullptr, k, v, out, HIFA4_BF16, lse, nullptr, 0, nullptr));
  EXPECT_FAIL(HIFA4_ERR_UNSUPPORTED, hifa4_attn_fwd_qraw(&dp, P(0x10000000), HIFA4_BF16, nullptr, k, v, out, HIFA4_BF16, lse, nullptr, 0, nullptr));
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_attn_fwd_qraw(&p, P(0x10000000), HIFA4_BF16, reinterpret_cast<float*>(0x70000004), k, v, out, HIFA4_BF16, lse, nullptr, 0, nullptr));
  EXPECT_OK(1, hifa4_attn_fwd_qraw(&p, P(0x10000000), HIFA4_BF16, reinterpret_cast<float*>(0x70000000), k, v, out, HIFA4_BF16, lse, nullptr, 0, nullptr));
  // ---- the allocation-free entry point
  EXPECT_OK(1, hifa4_attn_fwd_noalloc(&p, q, k, v, out, HIFA4_BF16, lse, nullptr));
  dp = params(1);
  EXPECT_OK(1, hifa4_attn_fwd_noalloc(&dp, q, k, v, out, HIFA4_BF16, lse, nullptr));
  hifa4_attn_params big = params(1);
  big.B = 64; big.Hkv = 8; big.Hq = 256; big.d = 256; big.Sk = 32768; big.kv_stride = 32768;
  EXPECT_FAIL(HIFA4_ERR_UNSUPPORTED, hifa4_attn_fwd_noalloc(&big, q, k, v, out, HIFA4_BF16, lse, nullptr));
  // ---- bf16 baseline
  p = params(1);
  p.kv_lens = reinterpret_cast<const int32_t*>(0xD0000000);
  EXPECT_FAIL(HIFA4_ERR_UNSUPPORTED, bf16_attn_fwd(&p, P(0x10000000), P(0x20000000), P(0x30000000), out, lse, nullptr, 0, nullptr));
  p = params(128); p.normaliser = 1;
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, bf16_attn_fwd(&p, P(0x10000000), P(0x20000000), P(0x30000000), out, lse, nullptr, 0, nullptr));
  p = params(128);
  EXPECT_OK(1, bf16_attn_fwd(&p, P(0x10000000), P(0x20000000), P(0x30000000), out, lse, nullptr, 0, nullptr));
  // ---- quantise
  const hifa4_mx_tensor qo = mx(0x80000000), ko = mx(0x90000000), vo = mx(0xA0000000);
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_quantize_qkv(nullptr, nullptr, nullptr, HIFA4_BF16, 1, 4, 2, 64, 64, 0, 128, nullptr, qo, ko, vo, nullptr));
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_quantize_qkv(P(0x10000004), nullptr, nullptr, HIFA4_BF16, 1, 4, 2, 64, 64, 0, 128, nullptr, qo, ko, vo, nullptr));
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_quantize_qkv(P(0x10000000), nullptr, nullptr, HIFA4_BF16, 1, 4, 2, 64, 64, 0, 128, nullptr, mx(0x10000000), ko, vo, nullptr));
  hifa4_mx_tensor bad_rule = qo;
  bad_rule.scale_rule = 4;
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_quantize_qkv(P(0x10000000), nullptr, nullptr, HIFA4_BF16, 1, 4, 2, 64, 64, 0, 128, nullptr, bad_rule, ko, vo, nullptr));
  EXPECT_FAIL(HIFA4_ERR_UNSUPPORTED, hifa4_quantize_qkv(P(0x10000000), nullptr, nullptr, HIFA4_BF16, 1, 4, 2, 64, 64, 0, 100, nullptr, qo, ko, vo, nullptr));
  EXPECT_OK(1, hifa4_quantize_qkv(P(0x10000000), P(0x20000000), P(0x30000000), HIFA4_BF16, 1, 4, 2, 64, 64, 0, 128, nullptr, qo, ko, vo, nullptr));
  hifa4_rope rope{reinterpret_cast<const float*>(0xB0000000), reinterpret_cast<const float*>(0xC0000000), 64, 0, 0};
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_quantize_qkv_rope(P(0x10000000), nullptr, nullptr, HIFA4_BF16, 1, 4, 2, 64, 64, 0, 128, nullptr, nullptr, qo, ko, vo, nullptr));
  rope.q_pos0 = 1;
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_quantize_qkv_rope(P(0x10000000), nullptr, nullptr, HIFA4_BF16, 1, 4, 2, 64, 64, 0, 128, nullptr, &rope, qo, ko, vo, nullptr));
  rope.q_pos0 = 0;
  EXPECT_OK(1, hifa4_quantize_qkv_rope(P(0x10000000), P(0x20000000), P(0x30000000), HIFA4_BF16, 1, 4, 2, 64, 64, 0, 128, nullptr, &rope, qo, ko, vo, nullptr));
  // ---- cache append
  const int32_t* lens = reinterpret_cast<const int32_t*>(0xD0000000);
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_kv_append(nullptr, P(0x20000000), P(0x30000000), HIFA4_BF16, 2, 8, 2, 1, 0, 128, lens, nullptr, nullptr, nullptr, P(0xE0000000), qo, ko, vo, nullptr));
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_kv_append(nullptr, P(0x20000000), P(0x30000000), HIFA4_BF16, 2, 8, 2, 1, 256, 128, nullptr, nullptr, nullptr, nullptr, P(0xE0000000), qo, ko, vo, nullptr));
  EXPECT_OK(1, hifa4_kv_append(P(0x10000000), P(0x20000000), P(0x30000000), HIFA4_BF16, 2, 8, 2, 1, 256, 128, lens, reinterpret_cast<int32_t*>(0xF0000000), nullptr, nullptr, P(0xE0000000), qo, ko, vo, nullptr));
  // ---- calibration
  const size_t cw = hifa4_smooth_calibrate_workspace_size(2, 128);
  CHECK(cw == 2u * 2 * 128 * 4);
  float* so = reinterpret_cast<float*>(0xB0000000);
  EXPECT_FAIL(HIFA4_ERR_WORKSPACE_TOO_SMALL, hifa4_smooth_calibrate(P(0x10000000), P(0x20000000), HIFA4_BF16, 1, 4, 2, 64, 128, nullptr, 0.5, so, ws, cw - 4, nullptr));
  EXPECT_FAIL(HIFA4_ERR_INVALID_ARGUMENT, hifa4_smooth_calibrate(P(0x10000000), P(0x20000000), HIFA4_BF16, 1, 4, 2, 64, 128, nullptr, NAN, so, ws, cw, nullptr));
  EXPECT_OK(1, hifa4_smooth_calibrate(P(0x10000000), P(0x20000000), HIFA4_BF16, 1, 4, 2, 64, 128, nullptr, 0.5, so, ws, cw, nullptr));
  // ---- status strings
  for (int s = -5; s <= 1; s++) CHECK(hifa4_status_string((hifa4_status)s) != nullptr);
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("abi driver: all checks passed, %d launches\n", g_launches);
  return 0;
}
