// api.cpp -- the C ABI declared in include/hifa4.h: argument validation,
// problem set-up and kernel dispatch.  Nothing is enqueued unless every
// argument has been checked; no device memory is ever allocated here.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "hifa4.h"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

// HIFA4_LOG set to a non-empty value other than "0": every attention launch
// prints its schedule (workgroups, key tile, decode split, workspace) to stderr.
bool log_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("HIFA4_LOG");
    return e && *e && std::strcmp(e, "0") != 0;
  }();
  return on;
}

hifa4_status fail(hifa4_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

hifa4_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return HIFA4_OK;
  return fail(HIFA4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
  const char* name;
  const void* p;
  int64_t bytes;
};

bool overlaps(const Span& a, const Span& b) {
  if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
  auto alo = reinterpret_cast<uintptr_t>(a.p), blo = reinterpret_cast<uintptr_t>(b.p);
  return alo < blo + (uintptr_t)b.bytes && blo < alo + (uintptr_t)a.bytes;
}

// Every output must be disjoint from every input and from every other output.
hifa4_status check_disjoint(const Span* in, int n_in, const Span* out, int n_out) {
  for (int i = 0; i < n_out; i++) {
    for (int j = 0; j < n_in; j++)
      if (overlaps(out[i], in[j]))
        return fail(HIFA4_ERR_INVALID_ARGUMENT, "output %s overlaps input %s", out[i].name,
                    in[j].name);
    for (int j = i + 1; j < n_out; j++)
      if (overlaps(out[i], out[j]))
        return fail(HIFA4_ERR_INVALID_ARGUMENT, "outputs %s and %s overlap", out[i].name,
                    out[j].name);
  }
  return HIFA4_OK;
}

bool supported_d(int d) { return d == 64 || d == 128 || d == 256; }

constexpr float kMaxRescaleThreshold = 64.0f;

int64_t row_codes_bytes(int64_t rows, int d) { return rows * (d / 2); }
int64_t row_scales_bytes(int64_t rows, int d) { return rows * (d / 32); }
int64_t col_blocks(int64_t heads, int cap) { return heads * ((cap + 31) / 32); }

// Kernel bias of a block-scale rule (hifa4_scale_rule); false for an unknown rule.
bool scale_bias(int32_t rule, uint32_t* bias) {
  if (rule == HIFA4_SCALE_OCP) *bias = hifa4::kScaleBiasOcp;
  else if (rule == HIFA4_SCALE_NOCLIP) *bias = hifa4::kScaleBiasNoClip;
  else return false;
  return true;
}

// Shared validation of the attention parameter block.
hifa4_status check_params(const hifa4_attn_params* p, int* cap, int* chunk) {
  if (!p) return fail(HIFA4_ERR_INVALID_ARGUMENT, "params is NULL");
  if (p->B < 0 || p->Sq < 0 || p->Sk < 0 || p->kv_stride < 0)
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "negative size (B=%d Sq=%d Sk=%d kv_stride=%d)", p->B,
                p->Sq, p->Sk, p->kv_stride);
  if (p->Hq <= 0 || p->Hkv <= 0 || p->Hq % p->Hkv != 0)
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "need Hq > 0, Hkv > 0 and Hq %% Hkv == 0 (Hq=%d Hkv=%d)",
                p->Hq, p->Hkv);
  if (!supported_d(p->d)) return fail(HIFA4_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128, 256)", p->d);
  if (!std::isfinite(p->sm_scale))
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "sm_scale is not finite");
  // P reaches 2^threshold and l up to Sk * 2^threshold in fp32: past 64 the
  // accumulators could overflow where exact arithmetic does not
  if (!std::isfinite(p->rescale_threshold) || p->rescale_threshold < 0.0f ||
      p->rescale_threshold > kMaxRescaleThreshold)
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "rescale_threshold must be finite and in [0, %g]",
                (double)kMaxRescaleThreshold);
  if (p->normaliser != 0 && p->normaliser != 1)
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "normaliser %d (0: P-Reordering, 1: direct)",
                p->normaliser);
  uint32_t bias;
  if (!scale_bias(p->scale_rule, &bias))
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "scale_rule %d (0: OCP, 1: no-clip)", p->scale_rule);
  *cap = p->kv_stride ? p->kv_stride : p->Sk;
  if (*cap < p->Sk) return fail(HIFA4_ERR_INVALID_ARGUMENT, "kv_stride %d < Sk %d", *cap, p->Sk);
  // a head's K / V codes are addressed through 32-bit buffer ranges and offsets
  if ((int64_t)(*cap + 31) / 32 * 32 * (p->d / 2) >= ((int64_t)1 << 31))
    return fail(HIFA4_ERR_UNSUPPORTED, "key capacity %d x d %d: a head's codes exceed 2^31 bytes",
                *cap, p->d);
  if (p->kv_lens && p->Sq != 1)
    return fail(HIFA4_ERR_UNSUPPORTED, "kv_lens is only supported with Sq == 1 (decode)");
  *chunk = 0;
  if (p->Sq == 1) {
    const int bn = hifa4::attn_block_n(p->d);
    if (p->decode_chunk < 0 || p->decode_chunk % bn)
      return fail(HIFA4_ERR_INVALID_ARGUMENT, "decode_chunk %d is not 0 or a positive multiple of %d",
                  p->decode_chunk, bn);
    // tile and piece indices of the decode schedule are 32-bit
    const int64_t pairs = (int64_t)p->B * p->Hkv;
    if (pairs * ((p->Sk + bn - 1) / bn) + pairs >= ((int64_t)1 << 31))
      return fail(HIFA4_ERR_UNSUPPORTED, "decode problem too large (B*Hkv*ceil(Sk/%d) >= 2^31)", bn);
    *chunk = p->decode_chunk;
  } else if (p->decode_chunk) {
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "decode_chunk is only meaningful with Sq == 1");
  }
  return HIFA4_OK;
}

// Decode partial rows: one per (piece, pair) run, at row piece + pair, so at
// most (pieces + pairs - 1) rows of G query heads x (m, l, 2 unused, acc[d]).
size_t decode_workspace(const hifa4_attn_params* p, int chunk) {
  if (p->Sq != 1) return 0;
  const int bn = hifa4::attn_block_n(p->d);
  const int64_t pairs = (int64_t)p->B * p->Hkv;
  const int64_t max_tiles = pairs * ((p->Sk + bn - 1) / bn);
  if (max_tiles == 0) return 0;
  const int64_t pieces = chunk > 0 ? (max_tiles + chunk / bn - 1) / (chunk / bn)
                                   : hifa4::attn_decode_waves(p->d);
  const int64_t rows = pieces + pairs - 1;
  return (size_t)rows * (p->Hq / p->Hkv) * (p->d + 4) * sizeof(float);
}

// Shared body of hifa4_attn_fwd (q_raw == NULL: Q as MX codes) and
// hifa4_attn_fwd_qraw (Q as bf16 / fp16 activations, quantised in the kernel).
static hifa4_status attn_fwd_impl(const hifa4_attn_params* p, hifa4_mx_tensor q, const void* q_raw,
                                  hifa4_dtype q_dtype, const float* smooth, hifa4_mx_tensor k,
                                  hifa4_mx_tensor v, void* out, hifa4_dtype out_dtype, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int cap, chunk;
  hifa4_status st = check_params(p, &cap, &chunk);
  if (st != HIFA4_OK) return st;
  if (q_raw) {
    if (p->Sq == 1)
      return fail(HIFA4_ERR_UNSUPPORTED, "Q from activations is supported for prefill (Sq > 1)");
    if (q_dtype != HIFA4_BF16 && q_dtype != HIFA4_FP16)
      return fail(HIFA4_ERR_INVALID_ARGUMENT, "q_dtype %d", (int)q_dtype);
    // the kernel reads the Q fields only through q_raw
    q.codes = static_cast<uint8_t*>(const_cast<void*>(q_raw));
    q.scales = q.codes;
  }
  if (out_dtype != HIFA4_BF16 && out_dtype != HIFA4_FP16)
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "out_dtype %d", (int)out_dtype);
  const int d = p->d;
  const int64_t rq = (int64_t)p->B * p->Hq * p->Sq;
  const int64_t rcap = (int64_t)p->B * p->Hkv * cap;
  if (rq == 0) return HIFA4_OK;
  const void* ptrs[] = {q.codes, q.scales, k.codes, k.scales, v.codes, v.scales, out};
  const char* names[] = {q_raw ? "q" : "q.codes", q_raw ? "q" : "q.scales", "k.codes", "k.scales",
                         "v.codes", "v.scales", "out"};
  for (int i = 0; i < 7; i++) {
    // with no key capacity (Sk == 0) the K / V buffers are empty and may be NULL
    const bool kv = i >= 2 && i < 6;
    if (!ptrs[i] && !(kv && rcap == 0)) return fail(HIFA4_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(HIFA4_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", names[i]);
  }
  if (lse && !aligned16(lse)) return fail(HIFA4_ERR_INVALID_ARGUMENT, "lse is not 16-byte aligned");
  if (smooth && !aligned16(smooth))
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "smooth is not 16-byte aligned");
  if (p->kv_lens && !aligned16(p->kv_lens))
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "kv_lens is not 16-byte aligned");
  const size_t need = decode_workspace(p, chunk);
  if (workspace_bytes < need)
    return fail(HIFA4_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes,
                need);
  if (need && !workspace) return fail(HIFA4_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (need && !aligned16(workspace))
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "workspace is not 16-byte aligned");
  const Span in[] = {{q_raw ? "q" : "q.codes", q.codes, q_raw ? rq * d * 2 : row_codes_bytes(rq, d)},
                     {q_raw ? "smooth" : "q.scales", q_raw ? (const void*)smooth : q.scales,
                      q_raw ? (smooth ? (int64_t)p->Hkv * d * 4 : 0) : row_scales_bytes(rq, d)},
                     {"k.codes", k.codes, row_codes_bytes(rcap, d)},
                     {"k.scales", k.scales, row_scales_bytes(rcap, d)},
                     {"v.codes", v.codes, col_blocks((int64_t)p->B * p->Hkv, cap) * d * 16},
                     {"v.scales", v.scales, col_blocks((int64_t)p->B * p->Hkv, cap) * d},
                     {"kv_lens", p->kv_lens, p->kv_lens ? (int64_t)p->B * 4 : 0}};
  const Span outs[] = {{"out", out, rq * d * 2},
                       {"lse", lse, lse ? rq * 4 : 0},
                       {"workspace", workspace, (int64_t)need}};
  st = check_disjoint(in, 7, outs, 3);
  if (st != HIFA4_OK) return st;

  hifa4::AttnArgs a = {};
  a.q_codes = q.codes;
  a.q_scales = q.scales;
  a.q_raw = static_cast<const uint16_t*>(q_raw);
  a.smooth = q_raw ? smooth : nullptr;
  a.q_raw_bf16 = q_dtype == HIFA4_BF16;
  a.k_codes = k.codes;
  a.k_scales = k.scales;
  a.v_codes = v.codes;
  a.v_scales = v.scales;
  a.out = out;
  a.lse = lse;
  a.kv_lens = p->kv_lens;
  a.partials = static_cast<float*>(workspace);
  a.B = p->B;
  a.Hq = p->Hq;
  a.Hkv = p->Hkv;
  a.Sq = p->Sq;
  a.Sk = p->Sk;
  a.d = d;
  a.cap = cap;
  a.causal = p->causal ? 1 : 0;
  a.out_fp16 = out_dtype == HIFA4_FP16;
  a.sm_scale = p->sm_scale > 0.0f ? p->sm_scale : 1.0f / std::sqrt((float)d);
  a.sm_log2 = a.sm_scale * 1.4426950408889634f;
  a.chunk = chunk;
  a.dec_waves = hifa4::attn_decode_waves(d);
  a.tau = p->rescale_threshold;
  a.direct_l = p->normaliser;
  scale_bias(p->scale_rule, &a.p_bias);  // checked in check_params
  a.q_bias = a.p_bias;
  if (log_enabled()) {
    const int bn = hifa4::attn_block_n(d);
    if (p->Sq == 1)
      std::fprintf(stderr,
                   "[hifa4] decode B=%d Hq=%d Hkv=%d d=%d cap=%d key tile %d, %s split "
                   "(%d-token runs), persistent grid %d waves, workspace %zu bytes%s\n",
                   p->B, p->Hq, p->Hkv, d, cap, bn, chunk ? "per-pair" : "balanced",
                   chunk, a.dec_waves, need, p->normaliser ? ", direct normaliser" : "");
    else
      std::fprintf(stderr,
                   "[hifa4] prefill B=%d Hq=%d Hkv=%d Sq=%d Sk=%d d=%d %s, %lld workgroups of "
                   "128 queries (4 waves), key tile %d, threshold %g, Q %s%s\n",
                   p->B, p->Hq, p->Hkv, p->Sq, p->Sk, d, p->causal ? "causal" : "non-causal",
                   (long long)((p->Sq + 127) / 128) * p->B * p->Hq, bn, (double)a.tau,
                   q_raw ? "quantised in the prologue" : "as MX codes",
                   p->normaliser ? ", direct normaliser" : "");
  }
  hipError_t e = p->Sq == 1 ? hifa4::launch_attn_decode_mxfp4(a, (hipStream_t)stream)
                            : hifa4::launch_attn_prefill_mxfp4(a, (hipStream_t)stream);
  if (e == hipErrorNotSupported)
    return fail(HIFA4_ERR_UNSUPPORTED, "no kernel for this configuration");
  return hip_status(e, "attention launch");
}

}  // namespace

extern "C" {

const char* hifa4_status_string(hifa4_status s) {
  switch (s) {
    case HIFA4_OK: return "ok";
    case HIFA4_ERR_INVALID_ARGUMENT: return "invalid argument";
    case HIFA4_ERR_UNSUPPORTED: return "unsupported";
    case HIFA4_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case HIFA4_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* hifa4_last_error(void) { return g_last_error.c_str(); }

namespace {

// Validation of the RoPE tables for tokens [q_pos0, q_pos0 + nq) and
// [k_pos0, k_pos0 + nk) (n = 0: that tensor is not rotated).
hifa4_status check_rope(const hifa4_rope* r, int d, int64_t nq, int64_t nk, Span* spans) {
  if (!r) return fail(HIFA4_ERR_INVALID_ARGUMENT, "rope is NULL");
  if (!r->cos || !r->sin) return fail(HIFA4_ERR_INVALID_ARGUMENT, "rope table is NULL");
  if (!aligned16(r->cos) || !aligned16(r->sin))
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "rope table is not 16-byte aligned");
  if (r->n_pos < 0 || r->q_pos0 < 0 || r->k_pos0 < 0)
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "negative rope position or table size");
  if (nq > 0 && (int64_t)r->q_pos0 + nq > r->n_pos)
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "query positions %d + %lld exceed the table (%d rows)",
                r->q_pos0, (long long)nq, r->n_pos);
  if (nk > 0 && (int64_t)r->k_pos0 + nk > r->n_pos)
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "key positions %d + %lld exceed the table (%d rows)",
                r->k_pos0, (long long)nk, r->n_pos);
  const int64_t bytes = (int64_t)r->n_pos * (d / 2) * 4;
  spans[0] = {"rope.cos", r->cos, bytes};
  spans[1] = {"rope.sin", r->sin, bytes};
  return HIFA4_OK;
}

hifa4_status quantize_impl(const void* q, const void* k, const void* v, hifa4_dtype in_dtype,
                           int32_t B, int32_t Hq, int32_t Hkv, int32_t Sq, int32_t Sk,
                           int32_t kv_stride, int32_t d, const float* smooth,
                           const hifa4_rope* rope, bool with_rope, hifa4_mx_tensor q_out,
                           hifa4_mx_tensor k_out, hifa4_mx_tensor v_out, void* stream) {
  if (in_dtype != HIFA4_BF16 && in_dtype != HIFA4_FP16)
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "in_dtype %d", (int)in_dtype);
  if (B < 0 || Sq < 0 || Sk < 0 || kv_stride < 0)
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "negative size");
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "need Hq > 0, Hkv > 0 and Hq %% Hkv == 0");
  if (!supported_d(d)) return fail(HIFA4_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128, 256)", d);
  const int cap = kv_stride ? kv_stride : Sk;
  if (cap < Sk) return fail(HIFA4_ERR_INVALID_ARGUMENT, "kv_stride %d < Sk %d", cap, Sk);
  if (!q && !k && !v) return fail(HIFA4_ERR_INVALID_ARGUMENT, "q, k and v are all NULL");
  struct Req {
    const char* name;
    const void* p;
  };
  const Req req[] = {{"q", q},           {"q_out.codes", q ? q_out.codes : nullptr},
                     {"q_out.scales", q ? q_out.scales : nullptr},
                     {"k", k},           {"k_out.codes", k ? k_out.codes : nullptr},
                     {"k_out.scales", k ? k_out.scales : nullptr},
                     {"v", v},           {"v_out.codes", v ? v_out.codes : nullptr},
                     {"v_out.scales", v ? v_out.scales : nullptr},
                     {"smooth", smooth}};
  for (const Req& r : req)
    if (r.p && !aligned16(r.p))
      return fail(HIFA4_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", r.name);
  if (q && (!q_out.codes || !q_out.scales))
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "q given but q_out has a NULL buffer");
  if (k && (!k_out.codes || !k_out.scales))
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "k given but k_out has a NULL buffer");
  if (v && (!v_out.codes || !v_out.scales))
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "v given but v_out has a NULL buffer");
  uint32_t qb = 0, kb = 0, vb = 0;
  if ((q && !scale_bias(q_out.scale_rule, &qb)) || (k && !scale_bias(k_out.scale_rule, &kb)) ||
      (v && !scale_bias(v_out.scale_rule, &vb)))
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "unknown scale_rule in an output (0: OCP, 1: no-clip)");

  const int64_t rq = (int64_t)B * Hq * Sq, rk = (int64_t)B * Hkv * Sk;
  const int64_t rcap = (int64_t)B * Hkv * cap;
  Span in[] = {{"q", q, rq * d * 2}, {"k", k, rk * d * 2}, {"v", v, rk * d * 2},
               {"smooth", smooth, smooth ? (int64_t)Hkv * d * 4 : 0}, {"", nullptr, 0},
               {"", nullptr, 0}};
  if (with_rope) {
    hifa4_status rs = check_rope(rope, d, q ? Sq : 0, k ? Sk : 0, in + 4);
    if (rs != HIFA4_OK) return rs;
  }
  const Span out[] = {
      {"q_out.codes", q ? q_out.codes : nullptr, row_codes_bytes(rq, d)},
      {"q_out.scales", q ? q_out.scales : nullptr, row_scales_bytes(rq, d)},
      {"k_out.codes", k ? k_out.codes : nullptr, row_codes_bytes(rcap, d)},
      {"k_out.scales", k ? k_out.scales : nullptr, row_scales_bytes(rcap, d)},
      {"v_out.codes", v ? v_out.codes : nullptr, col_blocks((int64_t)B * Hkv, cap) * d * 16},
      {"v_out.scales", v ? v_out.scales : nullptr, col_blocks((int64_t)B * Hkv, cap) * d}};
  hifa4_status st = check_disjoint(in, 6, out, 6);
  if (st != HIFA4_OK) return st;

  hifa4::QuantizeArgs a = {};
  if (with_rope) {
    a.rope_cos = rope->cos;
    a.rope_sin = rope->sin;
    a.q_pos0 = rope->q_pos0;
    a.k_pos0 = rope->k_pos0;
  }
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.smooth = smooth;
  a.q_codes = q_out.codes;
  a.q_scales = q_out.scales;
  a.q_bias = qb;
  a.k_bias = kb;
  a.v_bias = vb;
  a.k_codes = k_out.codes;
  a.k_scales = k_out.scales;
  a.v_codes = v_out.codes;
  a.v_scales = v_out.scales;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Sq = Sq;
  a.Sk = Sk;
  a.d = d;
  a.cap = cap;
  a.blocks_q = q ? rq * (d / 32) : 0;
  a.blocks_k = k ? rk * (d / 32) : 0;
  if (!q || rq == 0) a.q = nullptr;
  if (!k || rk == 0) a.k = nullptr;
  if (!v || rk == 0) a.v = nullptr;
  return hip_status(hifa4::launch_quantize_qkv(a, in_dtype == HIFA4_BF16, (hipStream_t)stream),
                    "quantize launch");
}

}  // namespace

hifa4_status hifa4_quantize_qkv(const void* q, const void* k, const void* v, hifa4_dtype in_dtype,
                                int32_t B, int32_t Hq, int32_t Hkv, int32_t Sq, int32_t Sk,
                                int32_t kv_stride, int32_t d, const float* smooth,
                                hifa4_mx_tensor q_out, hifa4_mx_tensor k_out,
                                hifa4_mx_tensor v_out, void* stream) {
  g_last_error.clear();
  return quantize_impl(q, k, v, in_dtype, B, Hq, Hkv, Sq, Sk, kv_stride, d, smooth, nullptr,
                       false, q_out, k_out, v_out, stream);
}

hifa4_status hifa4_quantize_qkv_rope(const void* q, const void* k, const void* v,
                                     hifa4_dtype in_dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                     int32_t Sq, int32_t Sk, int32_t kv_stride, int32_t d,
                                     const float* smooth, const hifa4_rope* rope,
                                     hifa4_mx_tensor q_out, hifa4_mx_tensor k_out,
                                     hifa4_mx_tensor v_out, void* stream) {
  g_last_error.clear();
  return quantize_impl(q, k, v, in_dtype, B, Hq, Hkv, Sq, Sk, kv_stride, d, smooth, rope, true,
                       q_out, k_out, v_out, stream);
}

hifa4_status hifa4_kv_append(const void* q, const void* k, const void* v, hifa4_dtype in_dtype,
                             int32_t B, int32_t Hq, int32_t Hkv, int32_t n_new, int32_t kv_stride,
                             int32_t d, const int32_t* kv_lens, int32_t* kv_lens_out,
                             const float* smooth, const hifa4_rope* rope, void* v_tail,
                             hifa4_mx_tensor q_out, hifa4_mx_tensor k_cache,
                             hifa4_mx_tensor v_cache, void* stream) {
  g_last_error.clear();
  if (in_dtype != HIFA4_BF16 && in_dtype != HIFA4_FP16)
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "in_dtype %d", (int)in_dtype);
  if (B < 0 || n_new < 0) return fail(HIFA4_ERR_INVALID_ARGUMENT, "negative size");
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "need Hq > 0, Hkv > 0 and Hq %% Hkv == 0");
  if (!supported_d(d)) return fail(HIFA4_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128, 256)", d);
  if (kv_stride <= 0) return fail(HIFA4_ERR_INVALID_ARGUMENT, "kv_stride (cache capacity) must be > 0");
  struct Req {
    const char* name;
    const void* p;
    bool needed;
  };
  const bool any_new = (int64_t)B * n_new > 0;
  const Req req[] = {{"k", k, any_new},
                     {"v", v, any_new},
                     {"kv_lens", kv_lens, true},
                     {"v_tail", v_tail, true},
                     {"k_cache.codes", k_cache.codes, true},
                     {"k_cache.scales", k_cache.scales, true},
                     {"v_cache.codes", v_cache.codes, true},
                     {"v_cache.scales", v_cache.scales, true},
                     {"q", q, false},
                     {"q_out.codes", q ? q_out.codes : nullptr, q != nullptr},
                     {"q_out.scales", q ? q_out.scales : nullptr, q != nullptr},
                     {"kv_lens_out", kv_lens_out, false},
                     {"smooth", smooth, false}};
  for (const Req& r : req) {
    if (r.needed && !r.p) return fail(HIFA4_ERR_INVALID_ARGUMENT, "%s is NULL", r.name);
    if (r.p && !aligned16(r.p))
      return fail(HIFA4_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", r.name);
  }
  uint32_t qb = 0, kb = 0, vb = 0;
  if ((q && !scale_bias(q_out.scale_rule, &qb)) || !scale_bias(k_cache.scale_rule, &kb) ||
      !scale_bias(v_cache.scale_rule, &vb))
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "unknown scale_rule in an output (0: OCP, 1: no-clip)");
  Span in[] = {{"q", q, (int64_t)B * Hq * n_new * d * 2},
               {"k", k, (int64_t)B * Hkv * n_new * d * 2},
               {"v", v, (int64_t)B * Hkv * n_new * d * 2},
               {"smooth", smooth, smooth ? (int64_t)Hkv * d * 4 : 0},
               {"kv_lens", kv_lens, (int64_t)B * 4},
               {"", nullptr, 0},
               {"", nullptr, 0}};
  if (rope) {
    if (!rope->cos || !rope->sin) return fail(HIFA4_ERR_INVALID_ARGUMENT, "rope table is NULL");
    if (!aligned16(rope->cos) || !aligned16(rope->sin))
      return fail(HIFA4_ERR_INVALID_ARGUMENT, "rope table is not 16-byte aligned");
    if (rope->n_pos < 1 || rope->q_pos0 < 0 || rope->k_pos0 < 0)
      return fail(HIFA4_ERR_INVALID_ARGUMENT, "rope needs n_pos >= 1 and positions >= 0");
    const int64_t top = (int64_t)(rope->q_pos0 > rope->k_pos0 ? rope->q_pos0 : rope->k_pos0) +
                        kv_stride + n_new;
    if (top > 0x7FFFFFFF) return fail(HIFA4_ERR_INVALID_ARGUMENT, "rope positions overflow");
    const int64_t bytes = (int64_t)rope->n_pos * (d / 2) * 4;
    in[5] = {"rope.cos", rope->cos, bytes};
    in[6] = {"rope.sin", rope->sin, bytes};
  }
  const int64_t rq = (int64_t)B * Hq * n_new, rcap = (int64_t)B * Hkv * kv_stride;
  const int64_t vblk = col_blocks((int64_t)B * Hkv, kv_stride);
  const Span out[] = {{"q_out.codes", q ? q_out.codes : nullptr, row_codes_bytes(rq, d)},
                      {"q_out.scales", q ? q_out.scales : nullptr, row_scales_bytes(rq, d)},
                      {"k_cache.codes", k_cache.codes, row_codes_bytes(rcap, d)},
                      {"k_cache.scales", k_cache.scales, row_scales_bytes(rcap, d)},
                      {"v_cache.codes", v_cache.codes, vblk * d * 16},
                      {"v_cache.scales", v_cache.scales, vblk * d},
                      {"kv_lens_out", kv_lens_out, (int64_t)B * 4},
                      {"v_tail", v_tail, (int64_t)B * Hkv * 32 * d * 2}};
  hifa4_status st = check_disjoint(in, 7, out, 8);
  if (st != HIFA4_OK) return st;

  hifa4::AppendArgs a = {};
  a.q = (q && rq > 0) ? static_cast<const uint16_t*>(q) : nullptr;
  a.k = any_new ? static_cast<const uint16_t*>(k) : nullptr;
  a.v = any_new ? static_cast<const uint16_t*>(v) : nullptr;
  a.smooth = smooth;
  if (rope) {
    a.rope_cos = rope->cos;
    a.rope_sin = rope->sin;
    a.n_pos = rope->n_pos;
    a.q_pos0 = rope->q_pos0;
    a.k_pos0 = rope->k_pos0;
  }
  a.lens = kv_lens;
  a.lens_out = kv_lens_out;
  a.v_tail = static_cast<uint16_t*>(v_tail);
  a.q_codes = q_out.codes;
  a.q_scales = q_out.scales;
  a.k_codes = k_cache.codes;
  a.k_scales = k_cache.scales;
  a.v_codes = v_cache.codes;
  a.v_scales = v_cache.scales;
  a.q_bias = qb;
  a.k_bias = kb;
  a.v_bias = vb;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.n_new = n_new;
  a.d = d;
  a.cap = kv_stride;
  return hip_status(hifa4::launch_kv_append(a, in_dtype == HIFA4_BF16, (hipStream_t)stream),
                    "kv append launch");
}

size_t hifa4_smooth_calibrate_workspace_size(int32_t Hkv, int32_t d) {
  if (Hkv <= 0 || !supported_d(d)) return 0;
  return (size_t)2 * Hkv * d * 4;
}

hifa4_status hifa4_smooth_calibrate(const void* q, const void* k, hifa4_dtype in_dtype,
                                    int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t d,
                                    const hifa4_rope* rope, double alpha, float* smooth_out,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (in_dtype != HIFA4_BF16 && in_dtype != HIFA4_FP16)
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "in_dtype %d", (int)in_dtype);
  if (B < 0 || S < 0) return fail(HIFA4_ERR_INVALID_ARGUMENT, "negative size");
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "need Hq > 0, Hkv > 0 and Hq %% Hkv == 0");
  if (!supported_d(d)) return fail(HIFA4_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128, 256)", d);
  if (!std::isfinite(alpha)) return fail(HIFA4_ERR_INVALID_ARGUMENT, "alpha is not finite");
  const int64_t rows_q = (int64_t)B * Hq * S, rows_k = (int64_t)B * Hkv * S;
  const bool any = rows_q > 0;
  if (any && (!q || !k)) return fail(HIFA4_ERR_INVALID_ARGUMENT, "q or k is NULL");
  if ((q && !aligned16(q)) || (k && !aligned16(k)))
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "q or k is not 16-byte aligned");
  if (!smooth_out || !aligned16(smooth_out))
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "smooth_out is NULL or not 16-byte aligned");
  const size_t need = hifa4_smooth_calibrate_workspace_size(Hkv, d);
  if (!workspace || !aligned16(workspace))
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "workspace is NULL or not 16-byte aligned");
  if (workspace_bytes < need)
    return fail(HIFA4_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes,
                need);
  Span in[] = {{"q", any ? q : nullptr, rows_q * d * 2},
               {"k", any ? k : nullptr, rows_k * d * 2},
               {"", nullptr, 0},
               {"", nullptr, 0}};
  if (rope) {
    hifa4_status rs = check_rope(rope, d, S, S, in + 2);
    if (rs != HIFA4_OK) return rs;
  }
  const Span out[] = {{"smooth_out", smooth_out, (int64_t)Hkv * d * 4},
                      {"workspace", workspace, (int64_t)need}};
  hifa4_status st = check_disjoint(in, 4, out, 2);
  if (st != HIFA4_OK) return st;

  hifa4::CalibrateArgs a = {};
  a.q = any ? static_cast<const uint16_t*>(q) : nullptr;
  a.k = any ? static_cast<const uint16_t*>(k) : nullptr;
  a.smooth = smooth_out;
  a.workspace = static_cast<uint32_t*>(workspace);
  if (rope) {
    a.rope_cos = rope->cos;
    a.rope_sin = rope->sin;
    a.q_pos0 = rope->q_pos0;
    a.k_pos0 = rope->k_pos0;
  }
  a.B = any ? B : 0;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.S = S;
  a.d = d;
  a.alpha = alpha;
  return hip_status(hifa4::launch_smooth_calibrate(a, in_dtype == HIFA4_BF16, (hipStream_t)stream),
                    "calibrate launch");
}

size_t hifa4_attn_workspace_size(const hifa4_attn_params* p) {
  int cap, chunk;
  const std::string saved = g_last_error;
  if (check_params(p, &cap, &chunk) != HIFA4_OK) {
    g_last_error = saved;
    return 0;
  }
  (void)cap;
  return decode_workspace(p, chunk);
}

hifa4_status hifa4_attn_schedule(const hifa4_attn_params* p, int32_t* block_n,
                                 int32_t* chunk_tokens) {
  g_last_error.clear();
  int cap, chunk;
  hifa4_status st = check_params(p, &cap, &chunk);
  if (st != HIFA4_OK) return st;
  if (block_n) *block_n = hifa4::attn_block_n(p->d);
  if (chunk_tokens) *chunk_tokens = chunk;
  return HIFA4_OK;
}

int32_t hifa4_attn_decode_piece_tiles(const hifa4_attn_params* p, int64_t total_tiles) {
  int cap, chunk;
  const std::string saved = g_last_error;
  if (check_params(p, &cap, &chunk) != HIFA4_OK || p->Sq != 1 || total_tiles < 0 ||
      total_tiles >= ((int64_t)1 << 31)) {
    g_last_error = saved;
    return 0;
  }
  return hifa4::decode_piece_tiles(chunk, hifa4::attn_decode_waves(p->d), (int)total_tiles);
}

hifa4_status hifa4_attn_fwd(const hifa4_attn_params* p, hifa4_mx_tensor q, hifa4_mx_tensor k,
                            hifa4_mx_tensor v, void* out, hifa4_dtype out_dtype, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return attn_fwd_impl(p, q, nullptr, HIFA4_BF16, nullptr, k, v, out, out_dtype, lse, workspace,
                       workspace_bytes, stream);
}

hifa4_status hifa4_attn_fwd_noalloc(const hifa4_attn_params* p, hifa4_mx_tensor q,
                                    hifa4_mx_tensor k, hifa4_mx_tensor v, void* out,
                                    hifa4_dtype out_dtype, float* lse, void* stream) {
  g_last_error.clear();
  int cap, chunk;
  hifa4_status st = check_params(p, &cap, &chunk);
  if (st != HIFA4_OK) return st;
  const size_t need = decode_workspace(p, chunk);
  static_assert(hifa4::kStaticScratchBytes == HIFA4_NOALLOC_SCRATCH_BYTES,
                "the header states the scratch size");
  if (need > hifa4::kStaticScratchBytes)
    return fail(HIFA4_ERR_UNSUPPORTED,
                "decode partials need %zu bytes, more than the %zu-byte device scratch of "
                "hifa4_attn_fwd_noalloc (use hifa4_attn_fwd with a workspace)",
                need, hifa4::kStaticScratchBytes);
  void* ws = nullptr;
  if (need) {
    const hipError_t e = hifa4::static_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, "device scratch lookup");
  }
  return attn_fwd_impl(p, q, nullptr, HIFA4_BF16, nullptr, k, v, out, out_dtype, lse, ws,
                       need ? hifa4::kStaticScratchBytes : 0, stream);
}

hifa4_status hifa4_attn_fwd_qraw(const hifa4_attn_params* p, const void* q, hifa4_dtype q_dtype,
                                 const float* smooth, hifa4_mx_tensor k, hifa4_mx_tensor v,
                                 void* out, hifa4_dtype out_dtype, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!q) {
    g_last_error.clear();
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "q is NULL");
  }
  return attn_fwd_impl(p, hifa4_mx_tensor{nullptr, nullptr}, q, q_dtype, smooth, k, v, out,
                       out_dtype, lse, workspace, workspace_bytes, stream);
}

hifa4_status bf16_attn_fwd(const hifa4_attn_params* p, const void* q, const void* k,
                           const void* v, void* out, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  g_last_error.clear();
  int cap, chunk;
  if (p && p->kv_lens) return fail(HIFA4_ERR_UNSUPPORTED, "bf16_attn_fwd takes no kv_lens");
  if (p && p->decode_chunk) return fail(HIFA4_ERR_INVALID_ARGUMENT, "bf16_attn_fwd takes no decode_chunk");
  if (p && p->normaliser)
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "bf16_attn_fwd has no normaliser variant");
  if (p && p->scale_rule)
    return fail(HIFA4_ERR_INVALID_ARGUMENT, "bf16_attn_fwd quantises nothing (scale_rule must be 0)");
  hifa4_attn_params pp;
  if (p) {
    pp = *p;
    pp.Sq = pp.Sq == 1 ? 2 : pp.Sq;  // the bf16 path has no split-K variant; validate as prefill
  }
  hifa4_status st = check_params(p ? &pp : nullptr, &cap, &chunk);
  if (st != HIFA4_OK) return st;
  const int d = p->d;
  // a head's bf16 K / V rows are addressed through 32-bit buffer ranges and offsets
  if ((int64_t)cap * d * 2 >= ((int64_t)1 << 31))
    return fail(HIFA4_ERR_UNSUPPORTED, "key capacity %d x d %d: a head's bf16 keys exceed 2^31 bytes",
                cap, d);
  const int64_t rq = (int64_t)p->B * p->Hq * p->Sq;
  const int64_t rcap = (int64_t)p->B * p->Hkv * cap;
  if (rq == 0) return HIFA4_OK;
  const void* ptrs[] = {q, k, v, out};
  const char* names[] = {"q", "k", "v", "out"};
  for (int i = 0; i < 4; i++) {
    if (!ptrs[i]) return fail(HIFA4_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(HIFA4_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", names[i]);
  }
  if (lse && !aligned16(lse)) return fail(HIFA4_ERR_INVALID_ARGUMENT, "lse is not 16-byte aligned");
  const Span in[] = {{"q", q, rq * d * 2}, {"k", k, rcap * d * 2}, {"v", v, rcap * d * 2}};
  const Span outs[] = {{"out", out, rq * d * 2}, {"lse", lse, lse ? rq * 4 : 0}};
  st = check_disjoint(in, 3, outs, 2);
  if (st != HIFA4_OK) return st;
  hifa4::Bf16AttnArgs a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.B = p->B;
  a.Hq = p->Hq;
  a.Hkv = p->Hkv;
  a.Sq = p->Sq;
  a.Sk = p->Sk;
  a.d = d;
  a.cap = cap;
  a.causal = p->causal ? 1 : 0;
  const float sm = p->sm_scale > 0.0f ? p->sm_scale : 1.0f / std::sqrt((float)d);
  a.sm_log2 = sm * 1.4426950408889634f;
  a.tau = p->rescale_threshold;
  hipError_t e = hifa4::launch_attn_prefill_bf16(a, (hipStream_t)stream);
  if (e == hipErrorNotSupported) return fail(HIFA4_ERR_UNSUPPORTED, "no kernel for this configuration");
  return hip_status(e, "bf16 attention launch");
}

}  // extern "C"
