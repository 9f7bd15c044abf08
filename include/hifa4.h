/*
 * hifa4.h -- C ABI of the MXFP4 FlashAttention library for MI355X (gfx950).
 *
 * Method: "HiFA4: Training-Free 4-bit FlashAttention on Ascend HIF4 NPUs for
 * LLM Inference", Abstract.  Both attention products (Q K^T and P V) run on
 * 4-bit block-scaled operands while the online-softmax state (running max m,
 * normaliser l) stays in higher precision (fp32 here); Smooth-QK rescales Q
 * and K per channel after RoPE (Q * s, K / s) with a calibration-static s;
 * P-Reordering sums the normaliser from the same quantised P_hat that feeds
 * the P V product, and that sum is fused into the P V matrix product.
 *
 * 4-bit format.  The pages name HIF4 but never define its bit layout, so the
 * library uses gfx950's native OCP MXFP4 as the stand-in: FP4 E2M1 elements
 * (2 per byte, element 2i in the low nibble), one E8M0 scale byte per 32
 * elements with exponent floor(log2(amax)) - 2 (byte = exponent + 127),
 * elements rounded to nearest-even and clamped to +-6.
 *
 * Conventions for every entry point:
 *   - all tensor pointers are DEVICE pointers owned by the caller, 16-byte
 *     aligned, contiguous in the layouts documented below;
 *   - `stream` is a hipStream_t (NULL = the default stream); every call only
 *     enqueues work on it and never synchronises;
 *   - the library never allocates device memory; scratch memory comes from the
 *     caller's `workspace` (sizes from hifa4_attn_workspace_size and
 *     hifa4_smooth_calibrate_workspace_size);
 *   - arguments are validated before anything is enqueued: on a negative
 *     status nothing was enqueued and hifa4_last_error() describes why;
 *   - a launch failure returns HIFA4_ERR_HIP; faults during execution surface
 *     at the caller's next synchronisation;
 *   - outputs must not overlap inputs or each other; inputs are read only (the
 *     one in/out buffer is hifa4_kv_append's v_tail, documented there);
 *   - NaN / Inf inputs are unsupported (results unspecified);
 *   - calls are reentrant; the only global state is the per-thread error text.
 */
#ifndef HIFA4_H_
#define HIFA4_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define HIFA4_API __attribute__((visibility("default")))
#else
#define HIFA4_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hifa4_status {
  HIFA4_OK = 0,
  HIFA4_ERR_INVALID_ARGUMENT = -1, /* null / misaligned pointer, bad size, overlap */
  HIFA4_ERR_UNSUPPORTED = -2,      /* valid request outside what the kernels implement */
  HIFA4_ERR_WORKSPACE_TOO_SMALL = -3,
  HIFA4_ERR_HIP = -4               /* the HIP runtime refused a launch */
} hifa4_status;

typedef enum hifa4_dtype { HIFA4_BF16 = 0, HIFA4_FP16 = 1 } hifa4_dtype;

/* An MXFP4 tensor: E2M1 codes and E8M0 scales, both device buffers.
 * Row layout (queries, keys), blocks of 32 along the head dim d:
 *   codes  [B][H][T][d/2]   scales [B][H][T][d/32]
 * Column layout (values), blocks of 32 consecutive tokens of one channel,
 * aligned to token 0, nblk = ceil(T / 32):
 *   codes  [B][H][nblk][d][16]  (token 32*j + 2i in the low nibble of byte i)
 *   scales [B][H][nblk][d]
 * T is Sq for queries and the token capacity kv_stride for keys / values. */
typedef struct hifa4_mx_tensor {
  uint8_t* codes;
  uint8_t* scales;
  int32_t scale_rule; /* hifa4_scale_rule the scales are computed with where this tensor is an
                         output (quantise, append); ignored where it is an attention input */
} hifa4_mx_tensor;

/* Shared-exponent rule of a 32-element block with maximum magnitude amax.
 * OCP: the OCP MX v1.0 exponent X = floor(log2(amax)) - 2 (clamped to the
 * E8M0 range; 0 for an all-zero block); elements above 6 * 2^X saturate to 6.
 * NOCLIP: X + 1 wherever amax > 6 * 2^X, else X: the smallest exponent at or
 * above the OCP one at which no element saturates.  The abstract of "HiFA4:
 * Training-Free 4-bit FlashAttention on Ascend HIF4 NPUs for LLM Inference"
 * names a 4-bit block format without defining it; OCP MXFP4 stands in for it
 * and NOCLIP is a variant of that stand-in. */
typedef enum hifa4_scale_rule { HIFA4_SCALE_OCP = 0, HIFA4_SCALE_NOCLIP = 1 } hifa4_scale_rule;

typedef struct hifa4_attn_params {
  int32_t B;          /* batch */
  int32_t Hq;         /* query heads */
  int32_t Hkv;        /* key/value heads; Hq % Hkv == 0, query head h reads kv head h / (Hq / Hkv) */
  int32_t Sq;         /* query tokens per sequence (1 selects the split-K decode path) */
  int32_t Sk;         /* key tokens per sequence (upper bound when kv_lens is given) */
  int32_t d;          /* head dim: 64, 128 or 256 */
  int32_t causal;     /* nonzero: key t visible to query i iff t <= i + L - Sq (bottom-right) */
  float sm_scale;     /* score scale applied to Q K^T; <= 0 selects 1/sqrt(d) */
  int32_t kv_stride;  /* token capacity of the K/V buffers (>= Sk); 0 means Sk */
  const int32_t* kv_lens; /* device [B] per-sequence key count L (<= Sk), or NULL (L = Sk);
                             only with Sq == 1 */
  int32_t decode_chunk;   /* decode run length in tokens (a multiple of the key tile): every
                             (sequence, KV head) is cut from its own key 0, independently of
                             the batch; or 0 for the balanced split over the library's
                             persistent grid (see hifa4_attn_fwd) */
  float rescale_threshold;  /* log2 units, in [0, 64].  A row's running max moves only when a key
                               tile's max exceeds it by more than this, so P may reach
                               2^threshold; 0 = move on every increase (P <= 1, the
                               FlashAttention-2 frame).  Exact attention is the same for any
                               value; P_hat (and so the MXFP4 result) depends on it. */
  int32_t normaliser;       /* 0: P-Reordering, the method (Abstract, P-Reordering): the
                               normaliser l = sum(P_hat) of the same 4-bit P_hat as the
                               numerator, from the P V MFMA through an all-ones value
                               column.  1: the non-reordered form the pages compare it
                               with: l = sum(P) of the fp32 P before quantisation, summed
                               on the vector ALU, numerator still P_hat V.  Must be 0 for
                               bf16_attn_fwd. */
  int32_t scale_rule;       /* hifa4_scale_rule of the blocks the attention call quantises
                               itself: P_hat, and Q in hifa4_attn_fwd_qraw.  Must be 0 for
                               bf16_attn_fwd. */
} hifa4_attn_params;

/*
 * Smooth-QK + MXFP4 quantisation of Q, K and V (one launch).
 * Abstract, Smooth-QK: Q' = Q * s and K' = K / s per channel, in fp32 with
 * IEEE round-to-nearest multiply and divide, applied to the post-RoPE
 * activations; s is static (from offline calibration).  V is not smoothed.
 * Inputs (device, in_dtype, contiguous):
 *   q [B][Hq][Sq][d], k [B][Hkv][Sk][d], v [B][Hkv][Sk][d]
 *   smooth: device fp32 [Hkv][d] (query head h uses row h / (Hq / Hkv)), or NULL for s = 1
 * Outputs: q_out in the row layout with T = Sq; k_out in the row layout and
 *   v_out in the column layout, both with T = kv_stride (>= Sk, 0 means Sk).
 *   Only tokens < Sk are written; the tail value block is zero-padded.  Each
 *   output's scales follow its own scale_rule (an unknown rule is an error).
 * Any of q / k / v may be NULL (with its output ignored) to skip that tensor.
 * d must be 64, 128 or 256.
 */
HIFA4_API hifa4_status hifa4_quantize_qkv(const void* q, const void* k, const void* v, hifa4_dtype in_dtype,
                                int32_t B, int32_t Hq, int32_t Hkv, int32_t Sq, int32_t Sk,
                                int32_t kv_stride, int32_t d, const float* smooth,
                                hifa4_mx_tensor q_out, hifa4_mx_tensor k_out,
                                hifa4_mx_tensor v_out, void* stream);

/*
 * Rotate-half rotary position embedding, the step Smooth-QK follows (the
 * Abstract places the smoothing after RoPE).  Channel pair (j, j + d/2),
 * j < d/2, of a token at position pos is rotated by the table entries
 * c = cos[pos][j], s = sin[pos][j]:
 *   x'[j] = x[j] * c - x[j + d/2] * s,   x'[j + d/2] = x[j + d/2] * c + x[j] * s
 * in fp32, each product rounded, then the sum (no fused multiply-add).  The
 * caller owns the tables (any base frequency or scaling), so the library does
 * not evaluate trigonometric functions.
 */
typedef struct hifa4_rope {
  const float* cos;  /* device fp32 [n_pos][d/2], 16-byte aligned */
  const float* sin;  /* device fp32 [n_pos][d/2], 16-byte aligned */
  int32_t n_pos;     /* rows of the tables */
  int32_t q_pos0;    /* position of query token 0 (the same for every batch entry) */
  int32_t k_pos0;    /* position of key token 0 (the same for every batch entry) */
} hifa4_rope;

/*
 * hifa4_quantize_qkv with RoPE: Q and K are rotated (rope, positions
 * q_pos0 + t and k_pos0 + t) in fp32, then smoothed and quantised exactly as
 * hifa4_quantize_qkv does; V is not rotated.  rope must not be NULL; the
 * positions of every token given (q_pos0 + Sq and k_pos0 + Sk, for the tensors
 * passed) must lie within [0, n_pos].  The tables are inputs (read only, not
 * overlapping the outputs).  Other arguments and errors as for
 * hifa4_quantize_qkv.
 */
HIFA4_API hifa4_status hifa4_quantize_qkv_rope(const void* q, const void* k, const void* v,
                                     hifa4_dtype in_dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                     int32_t Sq, int32_t Sk, int32_t kv_stride, int32_t d,
                                     const float* smooth, const hifa4_rope* rope,
                                     hifa4_mx_tensor q_out, hifa4_mx_tensor k_out,
                                     hifa4_mx_tensor v_out, void* stream);

/*
 * KV-cache append for decode: n_new tokens per sequence are added to an MXFP4
 * cache after RoPE and Smooth-QK, the steps the Abstract places before the
 * 4-bit attention (Smooth-QK after RoPE), at each sequence's own position.
 * Sequence b currently holds L_b = kv_lens[b] tokens; its new token i sits at
 * position L_b + i (RoPE table row q_pos0 / k_pos0 + L_b + i).
 *   q     [B][Hq][n_new][d] new queries, or NULL: rotated, smoothed (x s) and
 *         quantised to q_out, row layout with T = n_new (the decode Q of
 *         hifa4_attn_fwd when n_new == 1);
 *   k, v  [B][Hkv][n_new][d] new keys / values (NULL allowed when B * n_new == 0),
 *         k rotated, smoothed (/ s) and
 *         quantised into k_cache rows L_b .. L_b + n_new - 1; v into v_cache,
 *         where every value block the append touches is quantised again from
 *         the raw values of all its tokens, so after any sequence of appends
 *         the cache holds exactly what hifa4_quantize_qkv(_rope) of each whole
 *         sequence writes;
 *   v_tail  device, in_dtype [B][Hkv][32][d], IN/OUT: slot t % 32 holds the raw
 *         value of token t for the tokens of the last, partly filled value
 *         block (t >= 32 * floor(L_b / 32)); the call reads the slots below
 *         L_b % 32 and writes those of its new tokens in the block left open.
 *         Zero-initialise it with the cache (L_b == 0 reads nothing);
 *   kv_lens      device int32 [B], read only;
 *   kv_lens_out  device int32 [B] or NULL: receives min(L_b + n_new, kv_stride),
 *         ready for the next hifa4_attn_fwd decode call (must not be kv_lens);
 *   kv_stride    the cache capacity in tokens (> 0); k_cache / v_cache use the
 *         layouts of hifa4_mx_tensor with T = kv_stride; the blocks written
 *         (new rows, the requantised open value block, new Q) follow the
 *         scale_rule of q_out / k_cache / v_cache, which should be the rule
 *         the cache was built with for it to equal a one-shot quantisation;
 *   smooth, dtype as for hifa4_quantize_qkv; rope may be NULL (no rotation),
 *         else n_pos >= 1.
 * Lengths live on the device, so the host cannot check them: the caller
 * guarantees 0 <= L_b and L_b + n_new <= kv_stride (and within the tables).
 * The kernel clamps L_b to [0, kv_stride], writes no row past the capacity
 * and clamps table rows to n_pos - 1, so no access leaves the buffers, but the
 * result for such a sequence is unspecified.  One launch.
 */
HIFA4_API hifa4_status hifa4_kv_append(const void* q, const void* k, const void* v,
                             hifa4_dtype in_dtype, int32_t B, int32_t Hq, int32_t Hkv,
                             int32_t n_new, int32_t kv_stride, int32_t d,
                             const int32_t* kv_lens, int32_t* kv_lens_out,
                             const float* smooth, const hifa4_rope* rope, void* v_tail,
                             hifa4_mx_tensor q_out, hifa4_mx_tensor k_cache,
                             hifa4_mx_tensor v_cache, void* stream);

/* Bytes of device workspace hifa4_smooth_calibrate needs: 2 * Hkv * d * 4
 * (0 for Hkv <= 0 or an unsupported d). */
HIFA4_API size_t hifa4_smooth_calibrate_workspace_size(int32_t Hkv, int32_t d);

/*
 * Offline Smooth-QK calibration (Abstract, Smooth-QK: s is calibration-static):
 * from calibration activations q [B][Hq][S][d] and k [B][Hkv][S][d] (device,
 * in_dtype, contiguous, 16-byte aligned), optionally rotated first by rope
 * (NULL: the activations are already post-RoPE), writes smooth_out (device
 * fp32 [Hkv][d], the row layout hifa4_quantize_qkv takes):
 *   s[g][j] = (max |K[., g, ., j]| / max |Q[., h, ., j]|)^alpha
 * with the Q maximum over every query head h of g's group (h / (Hq / Hkv) ==
 * g), every batch entry and token; the ratio and the power in fp64, rounded
 * once to fp32 (the power is the device's fp64 pow, within an ulp of the
 * correctly rounded value, so s is within one fp32 ulp of the exact result).
 * s = 1 where either maximum is zero (including B * S == 0, when q and k may
 * be NULL).  alpha must be finite.  workspace: device, 16-byte aligned, at
 * least hifa4_smooth_calibrate_workspace_size(Hkv, d) bytes, not overlapping
 * q, k, the tables or smooth_out; its contents are overwritten.  Three
 * launches on stream (clear, maxima, finish).
 */
HIFA4_API hifa4_status hifa4_smooth_calibrate(const void* q, const void* k, hifa4_dtype in_dtype,
                                    int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t d,
                                    const hifa4_rope* rope, double alpha, float* smooth_out,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace hifa4_attn_fwd / bf16_attn_fwd need for p
 * (0 when none); returns 0 as well for invalid parameters. */
HIFA4_API size_t hifa4_attn_workspace_size(const hifa4_attn_params* p);

/*
 * Fused MXFP4 FlashAttention forward (prefill for Sq > 1, split-K decode for
 * Sq == 1).  Abstract: Q K^T and P V are 4-bit block-scaled products (gfx950
 * scaled-FP4 MFMA); m and l are fp32; P = exp(S - m_new) is quantised to
 * MXFP4 in registers (blocks of 32 keys aligned to key 0); the normaliser
 * l = sum(P_hat) comes out of the P V MFMA through an all-ones value column
 * (P-Reordering with the fused normaliser).  The running max is updated once
 * per key tile (width from hifa4_attn_schedule).
 * Decode (Sq == 1) splits the keys and merges the runs' (m, l, acc) with the
 * log-sum-exp rule; each run starts from a fresh softmax state.  A (sequence b,
 * KV head g) pair has ceil(L_b / 64) key tiles of 64, the last possibly partial.
 *   decode_chunk > 0 (per pair): every pair is cut from its own key 0 into runs
 *      of decode_chunk keys (the last one shorter): a fresh state starts at key
 *      t of a pair whenever t is a multiple of decode_chunk.  A sequence's
 *      result depends on its own length only, not on the rest of the batch.
 *   decode_chunk == 0 (balanced): the tiles of all pairs, pairs in order
 *      b * Hkv + g, are laid end to end, T tiles in all, and cut into pieces of
 *      hifa4_attn_decode_piece_tiles(p, T) tiles, one per wave of the
 *      persistent grid; a piece restarts where it crosses into the next pair.
 *      So a fresh state starts at key t of pair s whenever t == 0 or
 *      (first_tile(s) * 64 + t) is a multiple of 64 * piece_tiles, where
 *      first_tile(s) counts the tiles of every pair before s: the runs, and
 *      so P_hat and the output (within the tolerance of the method, not bit
 *      for bit), depend on the lengths of the other sequences in the batch.
 * q, k, v: MX tensors from hifa4_quantize_qkv (T = Sq for q, kv_stride for k, v;
 *      with a key capacity of 0 the k and v buffers are empty and may be NULL).
 * out: device [B][Hq][Sq][d] in out_dtype, O = acc / l (rows without any
 *      visible key are 0).  B * Hq * Sq == 0 enqueues nothing.
 * lse: device fp32 [B][Hq][Sq] natural-log sum-exp of the scaled scores
 *      (m + ln l; -inf for rows without a visible key), or NULL.
 * Limits: a head's K / V codes (kv_stride * d / 2 bytes, rounded up to whole value
 *      blocks) must stay below 2^31 bytes, else HIFA4_ERR_UNSUPPORTED.
 * workspace: device scratch of hifa4_attn_workspace_size(p) bytes (may be NULL if 0).
 *      Decode keeps there one fp32 partial row (m, l, 2 unused, acc[d]) per
 *      query head and per (piece, pair) run; prefill needs none.
 */
HIFA4_API hifa4_status hifa4_attn_fwd(const hifa4_attn_params* p, hifa4_mx_tensor q, hifa4_mx_tensor k,
                            hifa4_mx_tensor v, void* out, hifa4_dtype out_dtype, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device scratch behind hifa4_attn_fwd_noalloc, per GPU. */
#define HIFA4_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * hifa4_attn_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, arguments, layouts and errors as hifa4_attn_fwd, but
 * the decode partials live in a device array inside the library
 * (HIFA4_NOALLOC_SCRATCH_BYTES on every GPU it runs on, held until the process
 * ends) instead of a caller workspace.  The caller still passes inputs and
 * outputs.  A problem whose partials need more (hifa4_attn_workspace_size)
 * returns HIFA4_ERR_UNSUPPORTED with nothing enqueued; prefill needs none.
 * The call allocates nothing: the first call on a device looks up the array's
 * address there (the device current at the call must be the stream's).
 * Every call on one GPU shares that array, so calls that may overlap on one
 * GPU (other streams, other threads) race and must be serialised by the
 * caller; each call writes every partial it reads, so nothing needs clearing.
 */
HIFA4_API hifa4_status hifa4_attn_fwd_noalloc(const hifa4_attn_params* p, hifa4_mx_tensor q,
                                              hifa4_mx_tensor k, hifa4_mx_tensor v, void* out,
                                              hifa4_dtype out_dtype, float* lse, void* stream);

/*
 * hifa4_attn_fwd for prefill (Sq > 1) with Q given as activations: q is device
 * [B][Hq][Sq][d] in q_dtype (bf16 or fp16, contiguous, 16-byte aligned) and
 * smooth the same Smooth-QK factors hifa4_quantize_qkv takes (device fp32
 * [Hkv][d], or NULL for s = 1).  Each workgroup smooths and quantises its own
 * query rows to MXFP4 in registers with the arithmetic of hifa4_quantize_qkv
 * (Abstract, Smooth-QK), so the codes, and the output, are bit-identical to
 * hifa4_quantize_qkv followed by hifa4_attn_fwd; the caller quantises only K
 * and V, and Q is read once instead of being quantised, written and read
 * back.  Other arguments, layouts and errors as for hifa4_attn_fwd; Sq == 1
 * returns HIFA4_ERR_UNSUPPORTED.
 */
HIFA4_API hifa4_status hifa4_attn_fwd_qraw(const hifa4_attn_params* p, const void* q,
                                 hifa4_dtype q_dtype, const float* smooth, hifa4_mx_tensor k,
                                 hifa4_mx_tensor v, void* out, hifa4_dtype out_dtype, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * bf16 FlashAttention forward, the accuracy and latency baseline the pages
 * compare against (Abstract): bf16 MFMA products, fp32 softmax state, no
 * quantisation and no smoothing.  q [B][Hq][Sq][d], k / v [B][Hkv][kv_stride][d]
 * bf16 device; out bf16 [B][Hq][Sq][d]; lse as for hifa4_attn_fwd.
 * kv_lens must be NULL.  One head's keys (kv_stride * d * 2 bytes) must stay
 * below 2^31 bytes (HIFA4_ERR_UNSUPPORTED otherwise).
 */
HIFA4_API hifa4_status bf16_attn_fwd(const hifa4_attn_params* p, const void* q, const void* k,
                           const void* v, void* out, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream);

/* The key-tile width of the online-softmax frame (*block_n) and the decode
 * piece length the caller asked for (*chunk_tokens: p->decode_chunk, 0 for
 * the balanced split and for prefill) hifa4_attn_fwd uses for p.  P_hat
 * depends on the frame and the split (and on p->rescale_threshold), so a
 * reference implementation needs them. */
HIFA4_API hifa4_status hifa4_attn_schedule(const hifa4_attn_params* p, int32_t* block_n,
                                 int32_t* chunk_tokens);

/* Host query: tiles per decode piece for decode parameters p when the pairs
 * hold total_tiles key tiles in all (sum over b of Hkv * ceil(L_b / 64)):
 * p->decode_chunk / 64 if set, else max(1, ceil(total_tiles / W)) with W the
 * waves of the library's persistent decode grid for p->d.  Returns 0 for
 * invalid or prefill parameters (the error text is left unchanged). */
HIFA4_API int32_t hifa4_attn_decode_piece_tiles(const hifa4_attn_params* p, int64_t total_tiles);

/* Static text for a status code. */
HIFA4_API const char* hifa4_status_string(hifa4_status s);

/* Detail text of the last failing call on this thread ("" if none). */
HIFA4_API const char* hifa4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HIFA4_H_ */
