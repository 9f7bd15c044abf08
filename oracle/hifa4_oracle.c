/*
 * hifa4_oracle.c -- plain, slow CPU oracle for HiFA4-style MXFP4 FlashAttention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no source, header, table or helper
 * with the HIP library; the two meet only in the documented byte layouts.
 *
 * What it follows
 * ---------------
 * Method: "HiFA4: Training-Free 4-bit FlashAttention on Ascend HIF4 NPUs for
 * LLM Inference", Abstract (the only text the pages give for the method):
 *   - both attention products (Q K^T and P V) take 4-bit block-scaled operands,
 *     while the online-softmax state (running max m, normaliser l) is kept in
 *     higher precision than the operands;
 *   - Smooth-QK: a calibration-static per-channel rescale applied after RoPE,
 *     Q' = Q * s, K' = K / s, which leaves Q K^T unchanged in exact arithmetic;
 *   - P-Reordering: the normaliser is summed from the same quantised weights
 *     P_hat that feed the P V product (not from the unquantised P);
 *   - the inconsistent ("direct") form, normaliser from unquantised P, scales
 *     every output row coherently by sum(P_hat)/sum(P); its per-tile signed
 *     mismatch is the epsilon statistic.
 * Format: the pages never define the HIF4 bit layout, so the 4-bit format is
 * the OCP Microscaling (MX) v1.0 MXFP4 stand-in: FP4 E2M1 elements, one E8M0
 * shared scale per 32 elements, scale exponent = floor(log2(amax)) - 2 (2 is
 * the largest E2M1 exponent), elements rounded to nearest-even and clamped to
 * +-6 (the MX conversion rule from the same specification).
 *
 * Precision: every score, exponential, sum and accumulator is fp64.  The
 * smoothing multiply / divide is done in fp32 (IEEE round-to-nearest), because
 * that is where the method applies it: to the fp32 activations, before
 * quantisation.  Compile without -ffast-math and with -ffp-contract=off.
 *
 * Readings of the pages' gaps (each is also listed in the design notes):
 *   - FlashAttention-2 frame: P = exp(S - m_new), m_new includes the current
 *     key tile, so P <= 1; the key tile width bc is a parameter because P_hat
 *     depends on it; optionally a lazy frame (parameter tau): the running max
 *     moves only when a tile's row max exceeds it by more than tau (log2
 *     units), so P <= 2^tau (exact attention is the same either way);
 *   - P blocks are 32 consecutive keys aligned to absolute key index 0 (or to
 *     the split chunk start, itself a multiple of 32); masked keys give P = 0;
 *   - causal masking is bottom-right aligned: key t is visible to query i iff
 *     t <= i + L - Sq, with L the key count of that sequence;
 *   - a row with no visible key outputs 0 with lse = -inf;
 *   - split-K decode runs the online softmax from a fresh state on each chunk
 *     and merges the partial (m, l, acc) with the log-sum-exp rule; the chunk
 *     grid of a (sequence, KV head) may be shifted by a phase (a multiple of
 *     the key tile), so that a fresh state starts at every key t > 0 with
 *     (t + phase) % chunk == 0: any cut of a sequence into runs is a valid
 *     split, and the exact result does not depend on it.
 */
#define _USE_MATH_DEFINES
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* E2M1 element encoding (OCP MX v1.0, FP4 E2M1)                              */
/* ------------------------------------------------------------------------- */

/* Magnitudes of the eight E2M1 codes 0..7 (sign is bit 3). */
static const double kE2M1Magnitude[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e2m1_value(unsigned code) {
  double m = kE2M1Magnitude[code & 7u];
  return (code & 8u) ? -m : m;
}

/* Round y to the nearest E2M1 value; an exact tie goes to the even code
 * (the one whose mantissa bit is 0); magnitudes above 6 clamp to 6.
 * The sign bit of y is kept, also for results of magnitude zero. */
unsigned oracle_e2m1_encode(double y) {
  unsigned sign = signbit(y) ? 8u : 0u;
  double a = fabs(y);
  unsigned c;
  if (a >= 6.0) {
    c = 7u;
  } else {
    unsigned i = 0;
    while (i < 7u && kE2M1Magnitude[i + 1] <= a) i++;
    /* kE2M1Magnitude[i] <= a < kE2M1Magnitude[i + 1] */
    double below = a - kE2M1Magnitude[i];
    double above = kE2M1Magnitude[i + 1] - a;
    if (below < above)
      c = i;
    else if (above < below)
      c = i + 1;
    else
      c = (i % 2u == 0u) ? i : i + 1;
  }
  return sign | c;
}

/* Element-wise encode of n values (for sweeps of the rounding rule). */
void oracle_e2m1_encode_array(const double* y, long n, unsigned char* codes) {
  for (long i = 0; i < n; i++) codes[i] = (unsigned char)oracle_e2m1_encode(y[i]);
}

/* MX block quantisation of n <= 32 values x[k*stride].  Writes one 4-bit code
 * per element into codes[k] (value 0..15) and the dequantised value into
 * deq[k*deq_stride] when deq != NULL.  Returns the E8M0 scale byte.
 * Shared exponent, rule 0 (OCP MX v1.0): floor(log2(amax)) - 2, clamped to
 * [-127, 127]; a block of zeros gets exponent -127 (byte 0).  Elements above
 * 6 * 2^e then saturate to +-6 (amax in (6, 8) * 2^e).
 * Rule 1 (no-clip): the OCP exponent plus one whenever amax > 6 * 2^e, so that
 * amax / 2^e <= 6 and no element saturates; every block whose amax / 2^e is at
 * most 6 under the OCP rule keeps the OCP exponent and codes. */
unsigned oracle_mx_block(const double* x, int n, long stride, unsigned char* codes,
                         double* deq, long deq_stride, int rule) {
  double amax = 0.0;
  for (int k = 0; k < n; k++) {
    double a = fabs(x[k * stride]);
    if (a > amax) amax = a;
  }
  int e;
  if (amax == 0.0) {
    e = -127;
  } else {
    int ex;
    (void)frexp(amax, &ex); /* amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1 */
    e = ex - 1 - 2;
    if (e < -127) e = -127;
    if (rule == 1 && amax > ldexp(6.0, e)) e += 1;
    if (e > 127) e = 127;
  }
  for (int k = 0; k < n; k++) {
    unsigned c = oracle_e2m1_encode(ldexp(x[k * stride], -e));
    codes[k] = (unsigned char)c;
    if (deq) deq[k * deq_stride] = ldexp(oracle_e2m1_value(c), e);
  }
  return (unsigned)(e + 127);
}

/* ------------------------------------------------------------------------- */
/* Smooth-QK + quantisation of Q / K (blocks of 32 along the head dim)        */
/* ------------------------------------------------------------------------- */

/*
 * x:       fp32 [B][H][S][d] (the post-RoPE activations, exactly as stored)
 * smooth:  fp32 [Hs][d] or NULL (NULL = all ones); head h uses row h / group
 * divide:  0 -> x * s (queries), 1 -> x / s (keys); fp32 arithmetic
 * cap:     token capacity of the output buffers (>= S); row t of head (b, h)
 *          is written at ((b*H + h)*cap + t)
 * codes:   [B][H][cap][d/2]  element 2i in the low nibble, 2i+1 in the high
 * scales:  [B][H][cap][d/32] E8M0 bytes
 * deq:     double [B][H][S][d] or NULL; with quantise == 0 it receives the
 *          smoothed fp32 values unquantised and codes / scales are untouched.
 */
void oracle_quantize_rows(const float* x, int B, int H, int S, int d, const float* smooth,
                          int group, int divide, int cap, int quantise, unsigned char* codes,
                          unsigned char* scales, double* deq, int rule) {
  double* row = (double*)malloc(sizeof(double) * (size_t)d);
  unsigned char blk[32];
  for (int b = 0; b < B; b++)
    for (int h = 0; h < H; h++)
      for (int t = 0; t < S; t++) {
        const float* xr = x + (((size_t)b * H + h) * S + t) * d;
        const float* s = smooth ? smooth + (size_t)(h / group) * d : NULL;
        for (int j = 0; j < d; j++) {
          float v = xr[j];
          if (s) v = divide ? v / s[j] : v * s[j];
          row[j] = (double)v;
        }
        double* dq = deq ? deq + (((size_t)b * H + h) * S + t) * d : NULL;
        if (!quantise) {
          if (dq) memcpy(dq, row, sizeof(double) * (size_t)d);
          continue;
        }
        size_t orow = ((size_t)b * H + h) * cap + t;
        for (int j0 = 0; j0 < d; j0 += 32) {
          unsigned sc = oracle_mx_block(row + j0, 32, 1, blk, dq ? dq + j0 : NULL, 1, rule);
          scales[orow * (d / 32) + j0 / 32] = (unsigned char)sc;
          for (int k = 0; k < 32; k += 2)
            codes[orow * (d / 2) + (j0 + k) / 2] = (unsigned char)(blk[k] | (blk[k + 1] << 4));
        }
      }
  free(row);
}

/* ------------------------------------------------------------------------- */
/* The steps just before the path: RoPE and the offline Smooth-QK calibration  */
/* ------------------------------------------------------------------------- */

/*
 * Rotate-half rotary position embedding of rows x [rows][d] (fp32), the row r
 * being token t = r % S at position pos0 + t.  Channel pair (j, j + d/2),
 * j < d/2, is rotated by the angle whose cosine and sine are the tables'
 * entries [pos][j] (tables [n_pos][d/2], fp32, given by the caller):
 *   out[j]       = x[j] * cos - x[j + d/2] * sin
 *   out[j + d/2] = x[j + d/2] * cos + x[j] * sin
 * each product rounded to fp32, then the sum (no contraction).  The abstract
 * places Smooth-QK after RoPE; this is the rotation that precedes it.
 */
void oracle_rope_rows(const float* x, long rows, int S, int d, int pos0, const float* cosv,
                      const float* sinv, float* out) {
  const int half = d / 2;
  for (long r = 0; r < rows; r++) {
    const long pos = pos0 + r % S;
    const float* xr = x + (size_t)r * d;
    float* o = out + (size_t)r * d;
    for (int j = 0; j < half; j++) {
      const float c = cosv[(size_t)pos * half + j];
      const float sn = sinv[(size_t)pos * half + j];
      const float a = xr[j], b = xr[j + half];
      const float ac = a * c, bs = b * sn, bc = b * c, as = a * sn;
      o[j] = ac - bs;
      o[j + half] = bc + as;
    }
  }
}

/*
 * Offline Smooth-QK calibration (Abstract, Smooth-QK: calibration-static s):
 * per KV head g and channel j, s[g][j] = (max|K[., g, ., j]| / max|Q[., h, ., j]|)^alpha
 * with the Q maximum over every query head h of g's group (h / (Hq / Hkv) == g),
 * every batch entry and token; computed in fp64 and rounded to fp32 once.  A
 * zero maximum on either side gives s = 1.  q [B][Hq][S][d], k [B][Hkv][S][d].
 */
void oracle_smooth_calibrate(const double* q, const double* k, int B, int Hq, int Hkv, int S,
                             int d, double alpha, float* s_out) {
  const int G = Hq / Hkv;
  for (int g = 0; g < Hkv; g++)
    for (int j = 0; j < d; j++) {
      double qm = 0.0, km = 0.0;
      for (int b = 0; b < B; b++) {
        for (int t = 0; t < S; t++) {
          const double kv = fabs(k[(((size_t)b * Hkv + g) * S + t) * d + j]);
          if (kv > km) km = kv;
          for (int h = g * G; h < (g + 1) * G; h++) {
            const double qv = fabs(q[(((size_t)b * Hq + h) * S + t) * d + j]);
            if (qv > qm) qm = qv;
          }
        }
      }
      s_out[(size_t)g * d + j] = (qm > 0.0 && km > 0.0) ? (float)pow(km / qm, alpha) : 1.0f;
    }
}

/*
 * V quantisation: blocks of 32 consecutive tokens of one channel, aligned to
 * token 0; a partial tail block is padded with zeros (code 0) and its scale is
 * taken over the valid tokens only.
 * x:      fp32 [B][H][S][d]
 * codes:  [B][H][nblk][d][16], nblk = ceil(cap / 32); the 32 tokens of a
 *         block for one channel are 16 consecutive bytes, token 2i in the low
 *         nibble of byte i
 * scales: [B][H][nblk][d]
 * deq:    double [B][H][S][d] or NULL (with quantise == 0: the fp32 values)
 */
void oracle_quantize_v(const float* x, int B, int H, int S, int d, int cap, int quantise,
                       unsigned char* codes, unsigned char* scales, double* deq, int rule) {
  int nblk = (cap + 31) / 32;
  double col[32];
  double dqc[32];
  unsigned char blk[32];
  for (int b = 0; b < B; b++)
    for (int h = 0; h < H; h++) {
      const float* xh = x + ((size_t)b * H + h) * (size_t)S * d;
      double* dh = deq ? deq + ((size_t)b * H + h) * (size_t)S * d : NULL;
      for (int t0 = 0; t0 < S; t0 += 32) {
        int n = S - t0 < 32 ? S - t0 : 32;
        size_t blkrow = ((size_t)b * H + h) * nblk + t0 / 32;
        for (int c = 0; c < d; c++) {
          for (int k = 0; k < 32; k++) col[k] = k < n ? (double)xh[(size_t)(t0 + k) * d + c] : 0.0;
          if (!quantise) {
            if (dh)
              for (int k = 0; k < n; k++) dh[(size_t)(t0 + k) * d + c] = col[k];
            continue;
          }
          unsigned sc = oracle_mx_block(col, 32, 1, blk, dqc, 1, rule);
          scales[blkrow * d + c] = (unsigned char)sc;
          for (int k = 0; k < 32; k += 2)
            codes[(blkrow * d + c) * 16 + k / 2] = (unsigned char)(blk[k] | (blk[k + 1] << 4));
          if (dh)
            for (int k = 0; k < n; k++) dh[(size_t)(t0 + k) * d + c] = dqc[k];
        }
      }
    }
}

/* ------------------------------------------------------------------------- */
/* Attention: online softmax over key tiles with MXFP4 P_hat (P-Reordering)    */
/* ------------------------------------------------------------------------- */

typedef struct {
  int B, Hq, Hkv, Sq, Sk, d;
  int causal;
  double sm_scale; /* multiplies the raw dot products */
  int bc;          /* key tile width of the online-softmax frame */
  int chunk;       /* 0: one pass; > 0: split-K chunk length (multiple of bc) */
  int quant_p;     /* 1: P_hat = MXFP4(P) per 32-key block; 0: P_hat = P */
  int br;          /* query rows per epsilon tile */
  int nthreads;
  double tau;      /* lazy-rescale threshold in log2 units: the running max moves to a
                      tile's row max only if that exceeds it by more than tau; 0 gives the
                      FlashAttention-2 frame (P <= 1) */
  int p_rule;      /* block-scale rule of P_hat: 0 OCP, 1 no-clip (see oracle_mx_block) */
  double p_shift;  /* log2 units, normally 0: every P is taken as exp(S - m) * 2^p_shift.
                      Exact attention, O and the weights do not depend on it (the LSE is
                      corrected for it); P_hat does, where a P lies within 2^|p_shift| of a
                      rounding or block-exponent boundary of the 4-bit format.  A small
                      +-p_shift brackets an implementation that computes P in lower
                      precision (fp32 scores, a hardware exponential), so that its
                      quantisation decisions at such boundaries can be matched. */
} oracle_attn_cfg;

typedef struct {
  const oracle_attn_cfg* cfg;
  const double *q, *k, *v;
  const int32_t* kv_lens;
  const int32_t* chunk_phase; /* [B][Hkv] keys, or NULL (all 0) */
  const int64_t* rows; /* NULL: all rows, else flattened (b*Hq + h)*Sq + i */
  long n_rows;
  double *o, *lse, *o_naive, *l_out, *l_naive_out, *w;
  double *eps_sum, *eps_cnt, *ph_sum, *p_sum; /* [B][Hq][n_qt][n_kt] or NULL */
  int n_qt, n_kt;
  long next; /* work counter */
  pthread_mutex_t mu;
} attn_job;

/* One query row.  Scratch arrays are sized by the caller. */
static void attn_row(attn_job* J, int b, int h, int i, size_t out, double* S, double* P,
                     double* Ph, double* acc, double* acc_c, double* frame) {
  const oracle_attn_cfg* c = J->cfg;
  const int d = c->d;
  const int g = h / (c->Hq / c->Hkv);
  const int L = J->kv_lens ? J->kv_lens[b] : c->Sk;
  const size_t row = ((size_t)b * c->Hq + h) * c->Sq + i;
  const double* qr = J->q + row * d;
  const double* kh = J->k + ((size_t)b * c->Hkv + g) * (size_t)c->Sk * d;
  const double* vh = J->v + ((size_t)b * c->Hkv + g) * (size_t)c->Sk * d;
  double* wr = J->w ? J->w + out * (size_t)c->Sk : NULL;

  long last = (long)L - 1;
  if (c->causal && (long)i + L - c->Sq < last) last = (long)i + L - c->Sq;
  long nvis = last + 1; /* keys 0 .. nvis-1 are visible */

  double M = -INFINITY, lsum = 0.0, lnsum = 0.0;
  for (int j = 0; j < d; j++) acc[j] = 0.0;
  if (wr)
    for (int t = 0; t < c->Sk; t++) wr[t] = 0.0;

  long chunk = c->chunk > 0 ? c->chunk : (nvis > 0 ? nvis : 1);
  long phase = (c->chunk > 0 && J->chunk_phase) ? J->chunk_phase[(size_t)b * c->Hkv + g] : 0;
  for (long c0 = 0, cend; c0 < nvis; c0 = cend) {
    /* the next grid point after c0: the smallest t > c0 with (t + phase) % chunk == 0 */
    cend = ((c0 + phase) / chunk + 1) * chunk - phase;
    if (cend > nvis) cend = nvis;
    double m = -INFINITY, l = 0.0, ln = 0.0;
    for (int j = 0; j < d; j++) acc_c[j] = 0.0;
    for (long t0 = c0; t0 < cend; t0 += c->bc) {
      long t1 = t0 + c->bc < cend ? t0 + c->bc : cend; /* visible keys of this tile */
      long n = t1 - t0;
      double smax = -INFINITY;
      for (long t = t0; t < t1; t++) {
        const double* kr = kh + (size_t)t * d;
        double s = 0.0;
        for (int j = 0; j < d; j++) s += qr[j] * kr[j];
        s *= c->sm_scale;
        S[t - t0] = s;
        if (s > smax) smax = s;
      }
      /* the frame moves only for an increase of more than tau (log2 units) */
      double m_new = smax > m + c->tau * M_LN2 ? smax : m;
      double sumP = 0.0, sumPh = 0.0;
      for (long u = 0; u < n; u++) {
        P[u] = exp(S[u] - m_new + c->p_shift * M_LN2);
        sumP += P[u];
      }
      if (c->quant_p) {
        /* 32-key blocks aligned to absolute key index; keys past the visible
         * range contribute P = 0 to their block. */
        unsigned char codes[32];
        double blk[32], dq[32];
        for (long a0 = t0 - (t0 % 32); a0 < t1; a0 += 32) {
          for (int k = 0; k < 32; k++) {
            long t = a0 + k;
            blk[k] = (t >= t0 && t < t1) ? P[t - t0] : 0.0;
          }
          (void)oracle_mx_block(blk, 32, 1, codes, dq, 1, c->p_rule);
          for (int k = 0; k < 32; k++) {
            long t = a0 + k;
            if (t >= t0 && t < t1) Ph[t - t0] = dq[k];
          }
        }
      } else {
        for (long u = 0; u < n; u++) Ph[u] = P[u];
      }
      for (long u = 0; u < n; u++) sumPh += Ph[u];
      double alpha = exp(m - m_new); /* m = -inf on the first tile: alpha = 0 */
      l = alpha * l + sumPh;
      ln = alpha * ln + sumP;
      for (int j = 0; j < d; j++) acc_c[j] *= alpha;
      for (long u = 0; u < n; u++) {
        const double* vr = vh + (size_t)(t0 + u) * d;
        double p = Ph[u];
        for (int j = 0; j < d; j++) acc_c[j] += p * vr[j];
      }
      m = m_new;
      if (wr) {
        for (long u = 0; u < n; u++) {
          wr[t0 + u] = Ph[u];
          frame[t0 + u] = m_new;
        }
      }
      if (J->eps_sum && sumP > 0.0) {
        size_t ti = (((size_t)b * c->Hq + h) * J->n_qt + i / c->br) * J->n_kt + t0 / c->bc;
        J->eps_sum[ti] += sumPh / sumP - 1.0;
        J->eps_cnt[ti] += 1.0;
        J->ph_sum[ti] += sumPh;
        J->p_sum[ti] += sumP;
      }
    }
    /* log-sum-exp merge of this chunk into the row state */
    double Mn = M > m ? M : m;
    double a_old = exp(M - Mn), a_new = exp(m - Mn);
    lsum = a_old * lsum + a_new * l;
    lnsum = a_old * lnsum + a_new * ln;
    for (int j = 0; j < d; j++) acc[j] = a_old * acc[j] + a_new * acc_c[j];
    M = Mn;
  }

  double* o = J->o ? J->o + out * d : NULL;
  double* on = J->o_naive ? J->o_naive + out * d : NULL;
  if (nvis <= 0) {
    for (int j = 0; j < d; j++) {
      if (o) o[j] = 0.0;
      if (on) on[j] = 0.0;
    }
    if (J->lse) J->lse[out] = -INFINITY;
    if (J->l_out) J->l_out[out] = 0.0;
    if (J->l_naive_out) J->l_naive_out[out] = 0.0;
    return;
  }
  for (int j = 0; j < d; j++) {
    if (o) o[j] = acc[j] / lsum;
    if (on) on[j] = acc[j] / lnsum;
  }
  if (J->lse) J->lse[out] = M + log(lsum) - c->p_shift * M_LN2;
  if (J->l_out) J->l_out[out] = lsum;
  if (J->l_naive_out) J->l_naive_out[out] = lnsum;
  if (wr)
    for (long t = 0; t < nvis; t++) wr[t] = wr[t] * exp(frame[t] - M) / lsum;
}

static void* attn_worker(void* arg) {
  attn_job* J = (attn_job*)arg;
  const oracle_attn_cfg* c = J->cfg;
  size_t kmax = (size_t)c->Sk + 64;
  double* S = (double*)malloc(sizeof(double) * kmax);
  double* P = (double*)malloc(sizeof(double) * kmax);
  double* Ph = (double*)malloc(sizeof(double) * kmax);
  double* frame = (double*)malloc(sizeof(double) * kmax);
  double* acc = (double*)malloc(sizeof(double) * (size_t)c->d);
  double* acc_c = (double*)malloc(sizeof(double) * (size_t)c->d);
  /* Work unit: one (b, h, query tile of br rows) in full mode, so that a
   * tile's epsilon accumulators are owned by one thread; one row in subset
   * mode. */
  long n_units = J->rows ? J->n_rows : (long)c->B * c->Hq * J->n_qt;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    long u = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (u >= n_units) break;
    if (J->rows) {
      int64_t r = J->rows[u];
      int i = (int)(r % c->Sq);
      int h = (int)((r / c->Sq) % c->Hq);
      int b = (int)(r / ((int64_t)c->Sq * c->Hq));
      attn_row(J, b, h, i, (size_t)u, S, P, Ph, acc, acc_c, frame);
    } else {
      int qt = (int)(u % J->n_qt);
      int h = (int)((u / J->n_qt) % c->Hq);
      int b = (int)(u / ((long)J->n_qt * c->Hq));
      int i1 = (qt + 1) * c->br < c->Sq ? (qt + 1) * c->br : c->Sq;
      for (int i = qt * c->br; i < i1; i++)
        attn_row(J, b, h, i, ((size_t)b * c->Hq + h) * c->Sq + i, S, P, Ph, acc, acc_c, frame);
    }
  }
  free(S);
  free(P);
  free(Ph);
  free(frame);
  free(acc);
  free(acc_c);
  return NULL;
}

/*
 * q: double [B][Hq][Sq][d]; k, v: double [B][Hkv][Sk][d] (dequantised MXFP4
 * values, or exact values for the exact mode).  kv_lens: [B] or NULL.
 * chunk_phase: [B][Hkv] split phases in keys (multiples of bc below chunk), or
 * NULL; used only with chunk > 0.
 * rows: NULL for every row, else n_rows flattened row ids (b*Hq + h)*Sq + i.
 * Outputs (each may be NULL), indexed by row id, or by position in `rows`
 * when a subset is given: o, o_naive [rows][d]; lse, l, l_naive [rows];
 * w [rows][Sk] the final weight of every key (w . V = o);
 * eps_sum, eps_cnt, ph_sum, p_sum: [B][Hq][ceil(Sq/br)][ceil(Sk/bc)] per-tile
 * accumulators (full mode only; must be zeroed by the caller).
 * Returns 0, or -1 on a bad configuration.
 */
int oracle_attention(const oracle_attn_cfg* cfg, const double* q, const double* k,
                     const double* v, const int32_t* kv_lens, const int32_t* chunk_phase,
                     const int64_t* rows, long n_rows,
                     double* o, double* lse, double* o_naive, double* l_out, double* l_naive_out,
                     double* w, double* eps_sum, double* eps_cnt, double* ph_sum,
                     double* p_sum) {
  if (cfg->B < 0 || cfg->Hq <= 0 || cfg->Hkv <= 0 || cfg->Hq % cfg->Hkv || cfg->d <= 0 ||
      cfg->bc <= 0 || cfg->br <= 0 || cfg->Sq < 0 || cfg->Sk < 0)
    return -1;
  if (cfg->quant_p && cfg->bc % 32 && cfg->bc < cfg->Sk) return -1;
  if (cfg->chunk > 0 && cfg->chunk % cfg->bc) return -1;
  if (chunk_phase && cfg->chunk > 0)
    for (long i = 0; i < (long)cfg->B * cfg->Hkv; i++)
      if (chunk_phase[i] < 0 || chunk_phase[i] >= cfg->chunk || chunk_phase[i] % cfg->bc) return -1;
  attn_job J;
  memset(&J, 0, sizeof J);
  J.cfg = cfg;
  J.q = q;
  J.k = k;
  J.v = v;
  J.kv_lens = kv_lens;
  J.chunk_phase = chunk_phase;
  J.rows = rows;
  J.n_rows = n_rows;
  J.o = o;
  J.lse = lse;
  J.o_naive = o_naive;
  J.l_out = l_out;
  J.l_naive_out = l_naive_out;
  J.w = w;
  J.n_qt = (cfg->Sq + cfg->br - 1) / cfg->br;
  J.n_kt = (cfg->Sk + cfg->bc - 1) / cfg->bc;
  if (!rows) {
    J.eps_sum = eps_sum;
    J.eps_cnt = eps_cnt;
    J.ph_sum = ph_sum;
    J.p_sum = p_sum;
  }
  pthread_mutex_init(&J.mu, NULL);
  int nt = cfg->nthreads > 0 ? cfg->nthreads : 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
  for (int t = 0; t < nt; t++) pthread_create(&th[t], NULL, attn_worker, &J);
  for (int t = 0; t < nt; t++) pthread_join(th[t], NULL);
  free(th);
  pthread_mutex_destroy(&J.mu);
  return 0;
}

/*
 * The per-tile statistic of the inconsistent normaliser (Abstract, P-Reordering:
 * a normaliser from the unquantised P scales each output row by
 * sum(P_hat) / sum(P), and the pages report that mismatch per attention tile).
 * From the accumulators oracle_attention fills over n tiles:
 *   mean[t]   = eps_sum[t] / eps_cnt[t]: the mean over the tile's rows (those
 *               with sum(P) > 0 in that tile) of sum(P_hat) / sum(P) - 1;
 *   pooled[t] = ph_sum[t] / p_sum[t] - 1: the tile's total P_hat mass over its
 *               total P mass, minus one;
 * both NaN for a tile no row contributed to.
 */
void oracle_eps_tiles(const double* eps_sum, const double* eps_cnt, const double* ph_sum,
                      const double* p_sum, long n, double* mean, double* pooled) {
  for (long t = 0; t < n; t++) {
    if (eps_cnt[t] > 0.0) {
      mean[t] = eps_sum[t] / eps_cnt[t];
      pooled[t] = ph_sum[t] / p_sum[t] - 1.0;
    } else {
      mean[t] = NAN;
      pooled[t] = NAN;
    }
  }
}
