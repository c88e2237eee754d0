/*
 * csa2_oracle.c -- plain, slow, CPU reference for the CSA2 attention step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The product path never
 * calls it, and it shares no code, header, table or constant with the HIP
 * library: the two sides meet only at the bytes of the seeded synthetic inputs.
 *
 * Sources (cited by page title and section):
 *   [RN]   "Reading Notes of DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache
 *          Compression" -- section 3a (attention and its worked example),
 *          section 3f C2 (CSA2 steps 1-4), 3f C5 (SWA bounded replay).
 *   [WASTE] "DeepSeek-V4.1-Flash on WASTE" -- "What is new", 1. CSA2 (two KV
 *          sources in one softmax, attention sink, one 512-wide KV per token).
 *   [PLLM] PocketLLM "DeepSeek-V4.1-Flash" -- "The op layer" (finite score
 *          floor: an all-masked row is zeros), "The CSA2 attention layers"
 *          (window quantized to FP8 over 32 elements; a partial group emits
 *          nothing; compressed KV to FP4 with E4M3 scales over 16, indexer
 *          keys to FP4 with E8M0 scales over 32), "Correctness and precision"
 *          (-1 fills the unused top-k slots; ties), the FP4 quantizer notes
 *          (scale e4m3(amax / 6) with an amax floor of 6 * 2^-9; E8M0 scale
 *          2^round(log2(amax / 6)); round-to-even FP4 ties).
 *   [RN] 3f C4 (FP4 main KV cache: E2M1 grid, s = amax / 6 per 16 channels,
 *          codes round_E2M1(x / s), decode s * c; its worked example).
 *
 * Arithmetic: every floating-point step of the attention is fp64 over the
 * exactly decoded bf16 / fp8 inputs.  The indexer score is defined in fp32 by a
 * canonical sequential FMA chain (the pages do not fix the score precision;
 * this reading makes selected indices reproducible bit for bit), with an fp64
 * shadow and a rounding-error bound reported next to it.
 *
 * Every function validates its inputs and returns a negative code on refusal
 * (NaN/Inf input, reserved codes, bad sizes); it never aborts.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EBADARG (-1)
#define ORC_ENONFINITE (-2)
#define ORC_ENOMEM (-3)

enum { ORC_MODE_FULL = 0, ORC_MODE_REINDEX = 1, ORC_MODE_REUSE = 2, ORC_MODE_WINDOW = 3 };
enum { ORC_KV_BF16 = 0, ORC_KV_FP8 = 1, ORC_KV_FP4 = 2 };
enum { ORC_IDXK_F32 = 0, ORC_IDXK_MXFP4 = 1 };

/* ------------------------------------------------------------------------- */
/* O0: exact decoding of the storage formats                                  */
/* ------------------------------------------------------------------------- */

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits.  Returns -2 for
 * Inf/NaN, which the oracle refuses. */
int csa2o_bf16_to_f64(uint16_t b, double *out) {
  int s = (b >> 15) & 1, e = (b >> 7) & 0xFF, m = b & 0x7F;
  double v;
  if (e == 0xFF) return ORC_ENONFINITE;
  if (e == 0)
    v = ldexp((double)m, -133); /* 2^(1-127) * m/2^7 */
  else
    v = ldexp(1.0 + (double)m / 128.0, e - 127);
  *out = s ? -v : v;
  return ORC_OK;
}

/* FP8 E4M3 ("fn" variant: bias 7, no infinities, S.1111.111 is NaN), as used
 * for the sliding-window cache ([PLLM] "The CSA2 attention layers"). */
int csa2o_e4m3_to_f64(uint8_t c, double *out) {
  int s = (c >> 7) & 1, e = (c >> 3) & 0xF, m = c & 7;
  double v;
  if (e == 0xF && m == 7) return ORC_ENONFINITE;
  if (e == 0)
    v = ldexp((double)m, -9); /* subnormal: m/8 * 2^(1-7) */
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  *out = s ? -v : v;
  return ORC_OK;
}

/* UE8M0 block scale: an unsigned power of two 2^(e-127); 0xFF is NaN. */
int csa2o_ue8m0_to_f64(uint8_t e, double *out) {
  if (e == 0xFF) return ORC_ENONFINITE;
  *out = ldexp(1.0, (int)e - 127);
  return ORC_OK;
}

/* FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; magnitudes
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 ([RN] 3f C4).  `nib` is the low 4 bits. */
int csa2o_e2m1_to_f64(uint8_t nib, double *out) {
  int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
  double v = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, e - 1);
  *out = s ? -v : v;
  return ORC_OK;
}

/* Nearest E2M1 code to v, ties to the code with an even mantissa bit
 * ([PLLM] round-to-even FP4 ties); magnitudes above 6 are nearest to 6, so
 * they saturate there.  A zero magnitude is emitted as +0 (code 0). */
uint8_t csa2o_e2m1_encode(double v) {
  const double a = fabs(v);
  int best = 0, c;
  double bd = a;
  for (c = 1; c < 8; ++c) {
    double g, dist;
    csa2o_e2m1_to_f64((uint8_t)c, &g);
    dist = fabs(a - g);
    if (dist < bd || (dist == bd && (c & 1) == 0)) {
      bd = dist;
      best = c;
    }
  }
  return (uint8_t)((v < 0.0 && best != 0) ? (best | 8) : best);
}

/* Round a finite fp32 value to FP8 E4M3 (the "fn" variant), nearest-even,
 * saturating at +-448.  Written from the format: 3 fraction bits, exponent
 * bias 7, subnormal quantum 2^-9. */
int csa2o_f32_to_e4m3(float v, uint8_t *out) {
  double a = fabs((double)v), q, r;
  int e, ef;
  uint8_t sign = (v < 0.0f) ? 0x80 : 0x00;
  if (!isfinite(v)) return ORC_ENONFINITE;
  if (a >= 448.0) {
    *out = sign | 0x7E;
    return ORC_OK;
  }
  if (a < ldexp(1.0, -6)) {
    q = ldexp(1.0, -9); /* subnormal spacing */
  } else {
    frexp(a, &e);       /* a = f * 2^e, f in [0.5, 1) */
    q = ldexp(1.0, e - 1 - 3);
  }
  r = a / q; /* exact: q is a power of two */
  {
    double fl = floor(r), fr = r - fl;
    if (fr > 0.5 || (fr == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    r = fl * q;
  }
  if (r >= 448.0) r = 448.0;
  if (r == 0.0) {
    *out = sign;
    return ORC_OK;
  }
  if (r < ldexp(1.0, -6)) {
    *out = sign | (uint8_t)(r / ldexp(1.0, -9));
    return ORC_OK;
  }
  frexp(r, &e);
  ef = e - 1 + 7;
  *out = sign | (uint8_t)(ef << 3) | (uint8_t)((ldexp(r, -(e - 1)) - 1.0) * 8.0);
  return ORC_OK;
}

/* [RN] 3f C4 / [PLLM] FP4 quantizer of the main KV: per block of 16 values,
 * amax = max |x| (floored at 6 * 2^-9 so every scale is nonzero), the scale is
 * e4m3(amax / 6) with the division done in fp32, and each code is
 * round_E2M1(x / s) against that stored scale, the quotient taken in fp32.
 * Codes are packed two per byte, element 2i in the low nibble.  n must be a
 * multiple of 16; codes gets n/2 bytes, scales n/16 bytes. */
int csa2o_quant_fp4kv(const float *x, int64_t n, uint8_t *codes, uint8_t *scales) {
  int64_t b, i;
  if (n < 0 || (n % 16) != 0 || !x || !codes || !scales) return ORC_EBADARG;
  for (b = 0; b < n / 16; ++b) {
    const float *xb = x + 16 * b;
    float amax = 0.0f, s32, s;
    double sd;
    int rc;
    for (i = 0; i < 16; ++i) {
      if (!isfinite(xb[i])) return ORC_ENONFINITE;
      if (fabsf(xb[i]) > amax) amax = fabsf(xb[i]);
    }
    if (amax < 6.0f * 0.001953125f) amax = 6.0f * 0.001953125f;
    s32 = amax / 6.0f;
    if ((rc = csa2o_f32_to_e4m3(s32, &scales[b])) != ORC_OK) return rc;
    csa2o_e4m3_to_f64(scales[b], &sd);
    s = (float)sd; /* exact */
    for (i = 0; i < 16; i += 2) {
      const float q0 = xb[i] / s, q1 = xb[i + 1] / s;
      codes[8 * b + i / 2] = (uint8_t)(csa2o_e2m1_encode((double)q0) | (csa2o_e2m1_encode((double)q1) << 4));
    }
  }
  return ORC_OK;
}

/* [PLLM] MXFP4 quantizer of the indexer keys: per block of 32 values the
 * scale is 2^e with e = round(log2(amax / 6)) (amax / 6 taken in fp32), stored
 * as the E8M0 byte e + 127 and clamped to 1..254 (an all-zero block gets
 * 2^-126).  log2 of y = m 2^k (m in [1, 2)) rounds up exactly when m > sqrt 2,
 * i.e. m * m > 2, which is decided exactly in double; no tie is possible.
 * Codes are round_E2M1(x / 2^e), the quotient exact.  Packing as above;
 * codes gets n/2 bytes, scales n/32 bytes. */
int csa2o_quant_mxfp4(const float *x, int64_t n, uint8_t *codes, uint8_t *scales) {
  int64_t b, i;
  if (n < 0 || (n % 32) != 0 || !x || !codes || !scales) return ORC_EBADARG;
  for (b = 0; b < n / 32; ++b) {
    const float *xb = x + 32 * b;
    float amax = 0.0f, y;
    int e, k;
    for (i = 0; i < 32; ++i) {
      if (!isfinite(xb[i])) return ORC_ENONFINITE;
      if (fabsf(xb[i]) > amax) amax = fabsf(xb[i]);
    }
    y = amax / 6.0f;
    if (y == 0.0f) {
      e = -126;
    } else {
      double m = frexp((double)y, &k) * 2.0; /* y = m 2^(k-1), m in [1, 2) */
      e = (k - 1) + ((m * m > 2.0) ? 1 : 0);
    }
    if (e < -126) e = -126;
    if (e > 127) e = 127;
    scales[b] = (uint8_t)(e + 127);
    for (i = 0; i < 32; i += 2) {
      const double q0 = ldexp((double)xb[i], -e), q1 = ldexp((double)xb[i + 1], -e);
      codes[16 * b + i / 2] = (uint8_t)(csa2o_e2m1_encode(q0) | (csa2o_e2m1_encode(q1) << 4));
    }
  }
  return ORC_OK;
}

/* Decode n MXFP4 values (codes n/2 bytes, scales n/32 E8M0 bytes) to fp32;
 * exact (at most 2 significant bits times a power of two). */
int csa2o_dequant_mxfp4(const uint8_t *codes, const uint8_t *scales, int64_t n, float *out) {
  int64_t i;
  int rc;
  if (n < 0 || (n % 32) != 0 || !codes || !scales || !out) return ORC_EBADARG;
  for (i = 0; i < n; ++i) {
    double c, s;
    csa2o_e2m1_to_f64((uint8_t)((codes[i / 2] >> (4 * (i & 1))) & 15), &c);
    if ((rc = csa2o_ue8m0_to_f64(scales[i / 32], &s)) != ORC_OK) return rc;
    out[i] = (float)(c * s);
  }
  return ORC_OK;
}

/* Decode one KV row of d values.  bf16 rows are d uint16; fp8 rows are d codes
 * followed (in a separate plane) by d/32 UE8M0 scales, one per 32 values. */
static int decode_row(int kv_dtype, int d, const void *rows, const uint8_t *scales, int64_t r,
                      double *out) {
  int i, rc;
  if (kv_dtype == ORC_KV_BF16) {
    const uint16_t *p = (const uint16_t *)rows + (size_t)r * (size_t)d;
    for (i = 0; i < d; ++i)
      if ((rc = csa2o_bf16_to_f64(p[i], &out[i])) != ORC_OK) return rc;
    return ORC_OK;
  }
  if (kv_dtype == ORC_KV_FP8) {
    const uint8_t *p = (const uint8_t *)rows + (size_t)r * (size_t)d;
    const uint8_t *sc = scales + (size_t)r * (size_t)(d / 32);
    for (i = 0; i < d; ++i) {
      double code, scale;
      if ((rc = csa2o_e4m3_to_f64(p[i], &code)) != ORC_OK) return rc;
      if ((rc = csa2o_ue8m0_to_f64(sc[i / 32], &scale)) != ORC_OK) return rc;
      out[i] = code * scale; /* exact: a power-of-two scale */
    }
    return ORC_OK;
  }
  if (kv_dtype == ORC_KV_FP4) {
    /* FP4: d/2 bytes of E2M1 codes (element 2i low nibble) and d/16 E4M3 scales */
    const uint8_t *p = (const uint8_t *)rows + (size_t)r * (size_t)(d / 2);
    const uint8_t *sc = scales + (size_t)r * (size_t)(d / 16);
    for (i = 0; i < d; ++i) {
      double code, scale;
      csa2o_e2m1_to_f64((uint8_t)((p[i / 2] >> (4 * (i & 1))) & 15), &code);
      if ((rc = csa2o_e4m3_to_f64(sc[i / 16], &scale)) != ORC_OK) return rc;
      out[i] = code * scale; /* exact in double */
    }
    return ORC_OK;
  }
  return ORC_EBADARG;
}

/* ------------------------------------------------------------------------- */
/* O1: causal reachability ([RN] 3f C2 Step 1: block j covers m consecutive    */
/* tokens; [PLLM] a partial trailing group emits no entry yet).                */
/* ------------------------------------------------------------------------- */

/* With 0-based positions, compressed entry j stands for tokens j*m .. j*m+m-1
 * and exists once its last token is at or before the query position, so the
 * reachable entries are j < floor((pos+1)/m).  m == 0 (no compressed branch)
 * and window-only mode reach nothing.  The count is capped by the pool the
 * caller holds. */
int64_t csa2o_n_valid(int64_t pos, int32_t m, int32_t mode, int64_t pool_len) {
  int64_t n;
  if (pos < 0 || m < 0 || pool_len < 0) return ORC_EBADARG;
  if (m == 0 || mode == ORC_MODE_WINDOW) return 0;
  n = (pos + 1) / m;
  return n < pool_len ? n : pool_len;
}

/* ------------------------------------------------------------------------- */
/* Sliding window with the bounded-replay cut ([RN] 3f C2 Step 3: keys         */
/* t-w < u <= t; 3f C5: a window that would reach before the replay start s    */
/* begins at s instead).                                                       */
/* ------------------------------------------------------------------------- */
int csa2o_window_range(int64_t pos, int32_t w, int64_t replay_start, int64_t *lo, int64_t *count) {
  int64_t a;
  if (w < 0 || pos < replay_start) return ORC_EBADARG;
  a = pos - (int64_t)w + 1;
  if (a < replay_start) a = replay_start;
  *lo = a;
  *count = (w == 0) ? 0 : pos - a + 1;
  if (w == 0) *lo = pos + 1;
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* O3: indexer scores ([RN] 3f C2 Step 2, lightning-indexer form):             */
/*   sigma(j) = sum_h w_h * f(q_h . k_j),  f = ReLU (pages) or identity.       */
/* ------------------------------------------------------------------------- */

/* Canonical fp32 arithmetic for one candidate row `k` (d_i floats):
 *   per head h: acc = +0.0f; for i = 0..d_i-1: acc = fmaf(q[h][i], k[i], acc)
 *               f_h = relu ? (acc > 0 ? acc : +0) : acc
 *   s = +0.0f; for h = 0..h_i-1: s = fmaf(w_h, f_h, s)   (w_h = 1 when absent)
 *   -0.0 is mapped to +0.0.
 * The fp64 shadow evaluates the same expression in double, and `bound` is a
 * Higham-style bound on |s32 - s64|: recursive summation of exact products
 * errs by at most gamma_n * sum|terms| (gamma_n = n u / (1 - n u), u = 2^-24),
 * applied per head and once more over the head combination (f is 1-Lipschitz). */
static void score_one(int h_i, int d_i, const float *q, const float *w, int relu, const float *k,
                      float *s32, double *s64, double *bound) {
  const double u = ldexp(1.0, -24);
  double gam_d = (d_i * u) / (1.0 - d_i * u);
  double gam_h = (h_i * u) / (1.0 - h_i * u);
  float s = 0.0f;
  double t64 = 0.0, err = 0.0, abs_comb = 0.0;
  int h, i;
  for (h = 0; h < h_i; ++h) {
    const float *qh = q + (size_t)h * (size_t)d_i;
    float acc = 0.0f;
    double a64 = 0.0, absum = 0.0, f64;
    float f32, wh = w ? w[h] : 1.0f;
    for (i = 0; i < d_i; ++i) {
      acc = fmaf(qh[i], k[i], acc);
      a64 += (double)qh[i] * (double)k[i];
      absum += fabs((double)qh[i] * (double)k[i]);
    }
    f32 = relu ? (acc > 0.0f ? acc : 0.0f) : acc;
    f64 = relu ? (a64 > 0.0 ? a64 : 0.0) : a64;
    s = fmaf(wh, f32, s);
    t64 += (double)wh * f64;
    err += fabs((double)wh) * gam_d * absum;
    abs_comb += fabs((double)wh * (double)f32);
  }
  if (s == 0.0f) s = 0.0f; /* -0 -> +0 */
  *s32 = s;
  *s64 = t64;
  *bound = err * (1.0 + gam_h) + gam_h * abs_comb;
}

/* Scores for n candidates.  cand == NULL: candidate c is pool row c (Full
 * mode).  Otherwise candidate c is pool row cand[c] (Reindex mode).  keys are
 * the pool's index keys, row-major [rows, d_i].  Outputs are per candidate. */
int csa2o_index_scores(int32_t h_i, int32_t d_i, const float *q, const float *w, int32_t relu,
                       const float *keys, int64_t key_rows, const int32_t *cand, int64_t n,
                       float *s32, double *s64, double *bound) {
  int64_t c;
  int i;
  if (h_i < 1 || d_i < 1 || n < 0 || !q || !keys || !s32) return ORC_EBADARG;
  for (i = 0; i < h_i * d_i; ++i)
    if (!isfinite(q[i])) return ORC_ENONFINITE;
  if (w)
    for (i = 0; i < h_i; ++i)
      if (!isfinite(w[i])) return ORC_ENONFINITE;
  for (c = 0; c < n; ++c) {
    int64_t row = cand ? (int64_t)cand[c] : c;
    const float *k;
    double d64, b;
    if (row < 0 || row >= key_rows) return ORC_EBADARG;
    k = keys + (size_t)row * (size_t)d_i;
    for (i = 0; i < d_i; ++i)
      if (!isfinite(k[i])) return ORC_ENONFINITE;
    score_one(h_i, d_i, q, w, relu, k, &s32[c], &d64, &b);
    if (s64) s64[c] = d64;
    if (bound) bound[c] = b;
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* O4: top-K selection ([RN] 3f C2 Step 2: keep the K best; [PLLM]             */
/* "Correctness and precision": unused slots hold -1).  Order: score           */
/* descending, then pool index ascending (lowest index wins a tie); +0 and -0  */
/* compare equal.  Emitted in ascending pool-index order, padded with -1.      */
/* ------------------------------------------------------------------------- */
typedef struct {
  float s;
  int32_t pos;
} cand_t;

static int by_score_then_pos(const void *a, const void *b) {
  const cand_t *x = (const cand_t *)a, *y = (const cand_t *)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->pos < y->pos) ? -1 : (x->pos > y->pos);
}
static int by_pos(const void *a, const void *b) {
  const cand_t *x = (const cand_t *)a, *y = (const cand_t *)b;
  return (x->pos < y->pos) ? -1 : (x->pos > y->pos);
}

/* scores[c] belongs to pool row pos_of[c] (pos_of == NULL: row c).  Candidates
 * whose row is at or beyond n_valid are not eligible (Reindex lists may name
 * rows the query cannot reach yet). */
int csa2o_topk(const float *scores, const int32_t *pos_of, int64_t n, int64_t n_valid, int32_t k,
               int32_t *out) {
  cand_t *c;
  int64_t i, m = 0, take;
  if (n < 0 || k < 0 || !out || (n > 0 && !scores)) return ORC_EBADARG;
  c = (cand_t *)malloc(sizeof(cand_t) * (size_t)(n > 0 ? n : 1));
  if (!c) return ORC_ENOMEM;
  for (i = 0; i < n; ++i) {
    int32_t p = pos_of ? pos_of[i] : (int32_t)i;
    if (!isfinite(scores[i])) {
      free(c);
      return ORC_ENONFINITE;
    }
    if (p < 0 || p >= n_valid) continue;
    c[m].s = scores[i];
    c[m].pos = p;
    ++m;
  }
  qsort(c, (size_t)m, sizeof(cand_t), by_score_then_pos);
  take = m < k ? m : k;
  qsort(c, (size_t)take, sizeof(cand_t), by_pos);
  for (i = 0; i < k; ++i) out[i] = (i < take) ? c[i].pos : -1;
  free(c);
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* O6: single softmax over a set of entries ([RN] section 3a):                 */
/*   o = sum_e alpha_e v_e,  alpha_e = exp(s_e) / sum exp(s_e'),               */
/*   s_e = scale * <q, k_e>.  Written for separate K and V so the page's       */
/*   example (k != v) runs through it; CSA2 passes the same rows as both.      */
/* Attention sink ([WASTE] 1. CSA2): one per-head logit whose exponential      */
/* joins the denominator only.  No entries and no sink: o = 0, lse = -inf,     */
/* matching the finite-floor behaviour ([PLLM] "The op layer").                */
/* ------------------------------------------------------------------------- */
int csa2o_attend_core(int32_t h, int32_t d, int64_t e, const double *q, const double *kmat,
                      const double *vmat, const double *sink, double scale, double *out,
                      double *lse) {
  double *s;
  int64_t j;
  int hh, i;
  if (h < 1 || d < 1 || e < 0 || !q || !out || (e > 0 && (!kmat || !vmat))) return ORC_EBADARG;
  s = (double *)malloc(sizeof(double) * (size_t)(e > 0 ? e : 1));
  if (!s) return ORC_ENOMEM;
  for (hh = 0; hh < h; ++hh) {
    const double *qh = q + (size_t)hh * (size_t)d;
    double *oh = out + (size_t)hh * (size_t)d;
    double mx = -INFINITY, l = 0.0;
    for (j = 0; j < e; ++j) {
      double acc = 0.0;
      for (i = 0; i < d; ++i) acc += qh[i] * kmat[(size_t)j * (size_t)d + (size_t)i];
      s[j] = scale * acc;
      if (s[j] > mx) mx = s[j];
    }
    if (sink && sink[hh] > mx) mx = sink[hh];
    for (i = 0; i < d; ++i) oh[i] = 0.0;
    if (mx == -INFINITY) { /* nothing to attend to */
      if (lse) lse[hh] = -INFINITY;
      continue;
    }
    for (j = 0; j < e; ++j) {
      double p = exp(s[j] - mx);
      l += p;
      for (i = 0; i < d; ++i) oh[i] += p * vmat[(size_t)j * (size_t)d + (size_t)i];
    }
    if (sink) l += exp(sink[hh] - mx);
    for (i = 0; i < d; ++i) oh[i] /= l;
    if (lse) lse[hh] = mx + log(l);
  }
  free(s);
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Compressor ([RN] 3f C2 Step 1: each block of m consecutive tokens becomes   */
/* one entry, sum_u softmax_u(g_u) (.) c_u, the softmax over the block's tokens */
/* taken per channel; [PLLM] "The compressor": pooled in fp32, then RMS-normed; */
/* at ratio 1 there is no gate).  c and g are [n_groups * m][d] (g unused when  */
/* m == 1); out[j] = RMSNorm(pooled_j) = pooled / sqrt(mean(pooled^2) + eps)   */
/* (.) w, computed in double and rounded to fp32.                               */
/* ------------------------------------------------------------------------- */
int csa2o_compress(int64_t n_groups, int32_t m, int32_t d, const float *c, const float *g, const float *w,
                   double eps, float *out) {
  int64_t j;
  int i, u;
  double *pooled;
  if (n_groups < 0 || m < 1 || d < 1 || eps < 0.0 || (n_groups > 0 && (!c || !w || !out || (m > 1 && !g))))
    return ORC_EBADARG;
  pooled = (double *)malloc(sizeof(double) * (size_t)d);
  if (!pooled) return ORC_ENOMEM;
  for (j = 0; j < n_groups; ++j) {
    double ss = 0.0, r;
    for (i = 0; i < d; ++i) {
      if (m == 1) {
        pooled[i] = (double)c[(size_t)j * (size_t)d + (size_t)i];
      } else {
        double mx = -INFINITY, z = 0.0, acc = 0.0;
        for (u = 0; u < m; ++u) {
          const double gu = (double)g[((size_t)j * (size_t)m + (size_t)u) * (size_t)d + (size_t)i];
          if (gu > mx) mx = gu;
        }
        for (u = 0; u < m; ++u) {
          const size_t at = ((size_t)j * (size_t)m + (size_t)u) * (size_t)d + (size_t)i;
          const double e = exp((double)g[at] - mx);
          z += e;
          acc += e * (double)c[at];
        }
        pooled[i] = acc / z;
      }
      if (!isfinite(pooled[i])) {
        free(pooled);
        return ORC_ENONFINITE;
      }
      ss += pooled[i] * pooled[i];
    }
    r = 1.0 / sqrt(ss / (double)d + eps);
    for (i = 0; i < d; ++i) out[(size_t)j * (size_t)d + (size_t)i] = (float)(pooled[i] * r * (double)w[i]);
  }
  free(pooled);
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Compressor decode step ([RN] 3f C2 Step 1: entry j is the block of tokens   */
/* jm .. jm + m - 1, so it exists once its last token is in; [PLLM] "The CSA2  */
/* attention layers": the trailing partial group waits in state between      */
/* calls, and a step at a position that does not close a group emits nothing). */
/* One new token per sequence b at pos[b]: c_new[b], g_new[b] ([B][d]) become */
/* row u = pos[b] mod m of its state kv_state[b] / score_state[b] ([B][m][d]). */
/* When u == m - 1 the state holds the whole group: out[b] is the compressor  */
/* above over those m rows and emit_idx[b] = (pos[b] + 1) / m - 1; otherwise   */
/* out[b] is left as it was and emit_idx[b] = -1.  At m == 1 every token is   */
/* its own group (no gate, no state).                                          */
/* ------------------------------------------------------------------------- */
int csa2o_compress_step(int32_t B, int32_t m, int32_t d, const int64_t *pos, const float *c_new,
                        const float *g_new, float *kv_state, float *score_state, const float *w, double eps,
                        float *out, int32_t *emit_idx) {
  int32_t b;
  if (B < 0 || m < 1 || d < 1 || eps < 0.0) return ORC_EBADARG;
  if (B > 0 && (!pos || !c_new || !w || !out || !emit_idx || (m > 1 && (!g_new || !kv_state || !score_state))))
    return ORC_EBADARG;
  for (b = 0; b < B; ++b) {
    const int64_t p = pos[b];
    int64_t u;
    int rc;
    if (p < 0) return ORC_EBADARG;
    u = p % m;
    if (m == 1) {
      rc = csa2o_compress(1, 1, d, c_new + (size_t)b * (size_t)d, NULL, w, eps, out + (size_t)b * (size_t)d);
    } else {
      float *cs = kv_state + (size_t)b * (size_t)m * (size_t)d;
      float *gs = score_state + (size_t)b * (size_t)m * (size_t)d;
      memcpy(cs + (size_t)u * (size_t)d, c_new + (size_t)b * (size_t)d, sizeof(float) * (size_t)d);
      memcpy(gs + (size_t)u * (size_t)d, g_new + (size_t)b * (size_t)d, sizeof(float) * (size_t)d);
      if (u != m - 1) {
        emit_idx[b] = -1;
        continue;
      }
      rc = csa2o_compress(1, m, d, cs, gs, w, eps, out + (size_t)b * (size_t)d);
    }
    if (rc != ORC_OK) return rc;
    emit_idx[b] = (int32_t)((p + 1) / m - 1);
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Output de-rotation ([WASTE] "What is new", 1. CSA2: the rope dims of the    */
/* attention output are rotated by the conjugate of the query's rotation).     */
/* Each head's dims rope_off + 2i, rope_off + 2i + 1 (i < rope_dims / 2) form  */
/* a pair rotated by -pos * inv_freq[i]:                                        */
/*   (x, y) -> (x cos a + y sin a, -x sin a + y cos a),  a = pos * inv_freq[i]. */
/* The frequency table is the caller's (plain RoPE or a YaRN-scaled schedule). */
/* out [n_heads][d] is rotated in place (double arithmetic, rounded to fp32).  */
/* ------------------------------------------------------------------------- */
int csa2o_derotate(int32_t n_heads, int32_t d, int32_t rope_off, int32_t rope_dims, const double *inv_freq,
                   int64_t pos, float *out) {
  int h, i;
  if (n_heads < 1 || d < 1 || rope_off < 0 || rope_dims < 0 || (rope_dims % 2) != 0 || rope_off + rope_dims > d ||
      (rope_dims > 0 && !inv_freq) || !out)
    return ORC_EBADARG;
  for (h = 0; h < n_heads; ++h)
    for (i = 0; i < rope_dims / 2; ++i) {
      float *p = out + (size_t)h * (size_t)d + (size_t)rope_off + 2 * (size_t)i;
      const double a = (double)pos * inv_freq[i];
      const double x = p[0], y = p[1], cs = cos(a), sn = sin(a);
      p[0] = (float)(x * cs + y * sn);
      p[1] = (float)(-x * sn + y * cs);
    }
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Hierarchical candidate pool ([RN] 3f C3; [PLLM] "The CSA2 attention         */
/* layers", select_candidate_blocks): the Full layer's scores over the n       */
/* reachable entries are grouped into blocks of bs consecutive entries; a      */
/* block scores its best member; the pool is the top_blocks best blocks under  */
/* (block score descending, block index ascending), except that a block still  */
/* being filled (the last one, when n is not a multiple of bs) is always in    */
/* and takes one of the top_blocks places.  Output: the reachable entries of   */
/* the chosen blocks in ascending order, then -1 up to top_blocks * bs.        */
/* ------------------------------------------------------------------------- */
typedef struct {
  float s;
  int64_t blk;
} blk_t;

static int by_block_score(const void *a, const void *b) {
  const blk_t *x = (const blk_t *)a, *y = (const blk_t *)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->blk < y->blk) ? -1 : (x->blk > y->blk);
}

static int by_block_index(const void *a, const void *b) {
  const blk_t *x = (const blk_t *)a, *y = (const blk_t *)b;
  return (x->blk < y->blk) ? -1 : (x->blk > y->blk);
}

int csa2o_candidate_pool(const float *scores, int64_t n, int32_t bs, int32_t top_blocks, int32_t *out) {
  int64_t nblk, b, i, take, o = 0, nsort;
  int pinned;
  blk_t *v;
  if (n < 0 || bs < 1 || top_blocks < 1 || (n > 0 && !scores) || !out) return ORC_EBADARG;
  for (i = 0; i < n; ++i)
    if (isnan(scores[i])) return ORC_ENONFINITE;
  nblk = (n + bs - 1) / bs;
  pinned = (n % bs) != 0;
  v = (blk_t *)malloc(sizeof(blk_t) * (size_t)(nblk > 0 ? nblk : 1));
  if (!v) return ORC_ENOMEM;
  for (b = 0; b < nblk; ++b) {
    float m = -INFINITY;
    for (i = b * bs; i < (b + 1) * bs && i < n; ++i)
      if (scores[i] > m) m = scores[i];
    v[b].s = m;
    v[b].blk = b;
  }
  /* rank every block but the pinned one; the pinned block is the last */
  nsort = pinned ? nblk - 1 : nblk;
  qsort(v, (size_t)nsort, sizeof(blk_t), by_block_score);
  take = (int64_t)top_blocks - (pinned ? 1 : 0);
  if (take > nsort) take = nsort;
  if (take < 0) take = 0;
  if (pinned) v[take++] = v[nsort]; /* the pinned block: last, never sorted */
  qsort(v, (size_t)take, sizeof(blk_t), by_block_index);
  for (b = 0; b < take; ++b)
    for (i = v[b].blk * bs; i < (v[b].blk + 1) * bs && i < n; ++i) out[o++] = (int32_t)i;
  while (o < (int64_t)top_blocks * bs) out[o++] = -1;
  free(v);
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* O5 + O6 + O7 for one query: the entries are the win_len window rows (raw    */
/* KV) followed by the selected pool rows (compressed KV); one softmax runs    */
/* over their concatenation ([RN] 3f C2 Step 3; [WASTE] 1. CSA2).  The KV      */
/* vector is both key and value (one 512-wide KV per token, no separate V).    */
/* Window rows are win_rows[0 .. win_len-1]; selected entry idx (>= 0) is      */
/* pool row idx; -1 entries are skipped; other entries are attended as given   */
/* (duplicates count once per occurrence).                                     */
/* ------------------------------------------------------------------------- */
int csa2o_attend_query(int32_t h, int32_t d, int32_t kv_dtype, const uint16_t *q_bf16,
                       const void *win_rows, const uint8_t *win_scales, int64_t win_len,
                       const void *pool_rows, const uint8_t *pool_scales, int64_t pool_len,
                       const int32_t *sel, int32_t n_sel, const float *sink, double scale,
                       float *out, float *lse) {
  double *q = NULL, *kv = NULL, *o = NULL, *ls = NULL, *sk = NULL;
  int64_t e = 0, j;
  int rc = ORC_OK, i;
  if (h < 1 || d < 1 || win_len < 0 || n_sel < 0 || !q_bf16 || !out) return ORC_EBADARG;
  if (kv_dtype == ORC_KV_FP8 && (d % 32) != 0) return ORC_EBADARG;
  if (kv_dtype == ORC_KV_FP4 && (d % 16) != 0) return ORC_EBADARG;
  if (win_len > 0 && !win_rows) return ORC_EBADARG;
  if (!isfinite(scale)) return ORC_ENONFINITE;
  for (j = 0; j < n_sel; ++j) {
    if (sel[j] == -1) continue;
    if (sel[j] < 0 || sel[j] >= pool_len || !pool_rows) return ORC_EBADARG;
  }
  q = (double *)malloc(sizeof(double) * (size_t)h * (size_t)d);
  kv = (double *)malloc(sizeof(double) * (size_t)(win_len + n_sel + 1) * (size_t)d);
  o = (double *)malloc(sizeof(double) * (size_t)h * (size_t)d);
  ls = (double *)malloc(sizeof(double) * (size_t)h);
  if (sink) sk = (double *)malloc(sizeof(double) * (size_t)h);
  if (!q || !kv || !o || !ls || (sink && !sk)) {
    rc = ORC_ENOMEM;
    goto done;
  }
  for (i = 0; i < h * d; ++i)
    if ((rc = csa2o_bf16_to_f64(q_bf16[i], &q[i])) != ORC_OK) goto done;
  for (j = 0; j < win_len; ++j, ++e)
    if ((rc = decode_row(kv_dtype, d, win_rows, win_scales, j, kv + (size_t)e * (size_t)d)) != ORC_OK)
      goto done;
  for (j = 0; j < n_sel; ++j) {
    if (sel[j] == -1) continue;
    if ((rc = decode_row(kv_dtype, d, pool_rows, pool_scales, sel[j], kv + (size_t)e * (size_t)d)) !=
        ORC_OK)
      goto done;
    ++e;
  }
  if (sink)
    for (i = 0; i < h; ++i) {
      if (!isfinite(sink[i])) {
        rc = ORC_ENONFINITE;
        goto done;
      }
      sk[i] = sink[i];
    }
  if ((rc = csa2o_attend_core(h, d, e, q, kv, kv, sk, scale, o, ls)) != ORC_OK) goto done;
  for (i = 0; i < h * d; ++i) out[i] = (float)o[i]; /* round to nearest fp32 */
  if (lse)
    for (i = 0; i < h; ++i) lse[i] = (float)ls[i];
done:
  free(q);
  free(kv);
  free(o);
  free(ls);
  free(sk);
  return rc;
}

/* ------------------------------------------------------------------------- */
/* Selection for one query (O1-O4): candidates are the reachable pool rows     */
/* (Full) or the supplied list restricted to reachable rows (Reindex, [RN] 3f  */
/* C2 Step 4 and C3: a later layer scores only its allowed candidates).        */
/* Writes k indices; returns the number of scored candidates (>= 0) or a       */
/* negative error.  scores_out (optional, n floats) receives the fp32 scores   */
/* of the n scored candidates in candidate order.                              */
/* ------------------------------------------------------------------------- */
int64_t csa2o_select_query(int32_t mode, int64_t pos, int32_t m, int64_t pool_len, int32_t h_i,
                           int32_t d_i, const float *idx_q, const float *idx_w, int32_t relu,
                           const float *idx_k, const int32_t *cand, int64_t n_cand, int32_t k,
                           int32_t *out, float *scores_out) {
  int64_t nv = csa2o_n_valid(pos, m, mode, pool_len), n;
  float *s;
  int rc;
  if (nv < 0) return nv;
  if (mode != ORC_MODE_FULL && mode != ORC_MODE_REINDEX) return ORC_EBADARG;
  n = (mode == ORC_MODE_FULL) ? nv : n_cand;
  if (mode == ORC_MODE_REINDEX && n > 0 && !cand) return ORC_EBADARG;
  s = (float *)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
  if (!s) return ORC_ENOMEM;
  if (mode == ORC_MODE_REINDEX) {
    /* only reachable listed rows are scored; unreachable ones are dropped */
    int32_t *keep = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    int64_t c, nk = 0;
    if (!keep) {
      free(s);
      return ORC_ENOMEM;
    }
    for (c = 0; c < n; ++c)
      if (cand[c] >= 0 && cand[c] < nv) keep[nk++] = cand[c];
    rc = csa2o_index_scores(h_i, d_i, idx_q, idx_w, relu, idx_k, pool_len, keep, nk, s, NULL, NULL);
    if (rc == ORC_OK) rc = csa2o_topk(s, keep, nk, nv, k, out);
    if (rc == ORC_OK && scores_out) memcpy(scores_out, s, sizeof(float) * (size_t)nk);
    free(keep);
    free(s);
    return rc == ORC_OK ? nk : rc;
  }
  rc = csa2o_index_scores(h_i, d_i, idx_q, idx_w, relu, idx_k, pool_len, NULL, n, s, NULL, NULL);
  if (rc == ORC_OK) rc = csa2o_topk(s, NULL, n, nv, k, out);
  if (rc == ORC_OK && scores_out) memcpy(scores_out, s, sizeof(float) * (size_t)n);
  free(s);
  return rc == ORC_OK ? n : rc;
}

/* ------------------------------------------------------------------------- */
/* A batch of independent decode queries, each through the steps above in the */
/* pages' order: reachability -> (Full/Reindex) scores and top-K -> one        */
/* softmax over window rows and selected rows.  Reuse queries read their       */
/* selection from sel_io; Full/Reindex queries write theirs there.  Window     */
/* queries attend to their window only.  Layout per query b:                   */
/*   q [b][h][d] bf16;  window rows win_rows[win_row0[b] ..][d];               */
/*   pool rows / index keys start at pool_row0[b] and span pool_len[b] rows;   */
/*   idx_q [b][h_i][d_i];  idx_w [b][h_i] (or NULL);                           */
/*   Reindex lists cand_idx[cand_off[b] .. cand_off[b+1]) (pool-relative).     */
/* Index keys are fp32 [rows][d_i] (idx_kdtype 0) or MXFP4 (idx_kdtype 1:     */
/* codes [rows][d_i/2], E8M0 scales [rows][d_i/32]), decoded exactly to fp32   */
/* before the canonical score.  KV rows are bf16, fp8 (+ UE8M0 per 32) or FP4   */
/* (d/2 code bytes + E4M3 per 16).                                             */
/* Queries run in parallel (OpenMP) -- they share nothing.                     */
/* ------------------------------------------------------------------------- */
int csa2o_decode_batch(int32_t nb, int32_t h, int32_t d, int32_t k, int32_t h_i, int32_t d_i,
                       int32_t relu, int32_t kv_dtype, double scale, const int64_t *pos,
                       const int32_t *mode, const int32_t *ratio, const int64_t *win_row0,
                       const int32_t *win_len, const int64_t *pool_row0, const int32_t *pool_len,
                       const int64_t *cand_off, const int32_t *cand_idx, const uint16_t *q,
                       const void *win_rows, const uint8_t *win_scales, const void *pool_rows,
                       const uint8_t *pool_scales, const float *idx_q, const float *idx_w,
                       int32_t idx_kdtype, const void *idx_k, const uint8_t *idx_k_scales,
                       const float *sink, int32_t *sel_io, float *out, float *lse) {
  int32_t b;
  int err = ORC_OK;
  /* bytes per KV row and scale bytes per row */
  size_t rb = (kv_dtype == ORC_KV_FP8) ? (size_t)d : (kv_dtype == ORC_KV_FP4) ? (size_t)d / 2 : 2 * (size_t)d;
  size_t sb = (kv_dtype == ORC_KV_FP8) ? (size_t)d / 32 : (kv_dtype == ORC_KV_FP4) ? (size_t)d / 16 : 0;
  if (idx_kdtype != ORC_IDXK_F32 && idx_kdtype != ORC_IDXK_MXFP4) return ORC_EBADARG;
  if (idx_kdtype == ORC_IDXK_MXFP4 && ((d_i % 32) != 0 || !idx_k_scales)) return ORC_EBADARG;
#pragma omp parallel for schedule(dynamic, 1)
  for (b = 0; b < nb; ++b) {
    int rc = ORC_OK;
    int32_t *sel = sel_io + (size_t)b * (size_t)k;
    const uint8_t *wr = (const uint8_t *)win_rows + (size_t)win_row0[b] * rb;
    const uint8_t *ws = win_scales ? win_scales + (size_t)win_row0[b] * sb : NULL;
    const uint8_t *pr = (const uint8_t *)pool_rows + (size_t)pool_row0[b] * rb;
    const uint8_t *ps = pool_scales ? pool_scales + (size_t)pool_row0[b] * sb : NULL;
    int32_t nsel = k;
    if (mode[b] == ORC_MODE_FULL || mode[b] == ORC_MODE_REINDEX) {
      const int32_t *cl = (mode[b] == ORC_MODE_REINDEX) ? cand_idx + cand_off[b] : NULL;
      int64_t nc = (mode[b] == ORC_MODE_REINDEX) ? cand_off[b + 1] - cand_off[b] : 0;
      const float *keys = NULL;
      float *dec = NULL;
      int64_t r;
      if (idx_kdtype == ORC_IDXK_F32) {
        keys = (const float *)idx_k + (size_t)pool_row0[b] * (size_t)d_i;
      } else {
        dec = (float *)malloc(sizeof(float) * (size_t)(pool_len[b] > 0 ? pool_len[b] : 1) * (size_t)d_i);
        if (!dec) {
          rc = ORC_ENOMEM;
        } else {
          rc = csa2o_dequant_mxfp4((const uint8_t *)idx_k + (size_t)pool_row0[b] * (size_t)(d_i / 2),
                                   idx_k_scales + (size_t)pool_row0[b] * (size_t)(d_i / 32),
                                   (int64_t)pool_len[b] * d_i, dec);
          keys = dec;
        }
      }
      r = (rc == ORC_OK)
              ? csa2o_select_query(mode[b], pos[b], ratio[b], pool_len[b], h_i, d_i,
                                   idx_q + (size_t)b * (size_t)(h_i * d_i),
                                   idx_w ? idx_w + (size_t)b * (size_t)h_i : NULL, relu, keys, cl, nc, k, sel, NULL)
              : rc;
      free(dec);
      if (r < 0) rc = (int)r;
    } else if (mode[b] == ORC_MODE_WINDOW) {
      nsel = 0;
    } else if (mode[b] != ORC_MODE_REUSE) {
      rc = ORC_EBADARG;
    }
    if (rc == ORC_OK)
      rc = csa2o_attend_query(h, d, kv_dtype, q + (size_t)b * (size_t)(h * d), wr, ws, win_len[b], pr,
                              ps, pool_len[b], sel, nsel, sink, scale,
                              out + (size_t)b * (size_t)(h * d), lse ? lse + (size_t)b * (size_t)h : NULL);
    if (rc != ORC_OK) {
#pragma omp critical
      err = rc;
    }
  }
  return err;
}

/* ------------------------------------------------------------------------- */
/* One prefill chunk: T queries of one sequence at consecutive positions       */
/* pos0 .. pos0+T-1 ([RN] 3f C2 Steps 1-4), sharing the sequence's pool, index */
/* keys and raw window rows.  Raw row r holds position win_pos0 + r; win_pos0  */
/* is also the replay start, so the query at p reads the rows of positions     */
/* window_range(p, w, win_pos0) ([RN] 3f C5: the window never reaches before   */
/* the replay start).  The chunk has one mode; Reindex lists are per query     */
/* (cand_idx[cand_off[t] .. cand_off[t+1]]).  Only the queries qs[0..nq-1] are */
/* run; outputs are indexed by i < nq: sel_io [nq][k] (read for Reuse, written */
/* for Full / Reindex), out [nq][h][d], lse [nq][h].  q, idx_q and idx_w are   */
/* indexed by the query's t.  Index keys: fp32 [pool_len][d_i], or MXFP4       */
/* decoded exactly to fp32 first (idx_kdtype as for the decode batch).         */
/* ------------------------------------------------------------------------- */
int csa2o_prefill_chunk(int32_t nq, const int32_t *qs, int64_t pos0, int32_t mode, int32_t m, int64_t pool_len,
                        int64_t win_pos0, int64_t n_win_rows, int32_t w, int32_t h, int32_t d, int32_t k,
                        int32_t h_i, int32_t d_i, int32_t relu, int32_t kv_dtype, double scale,
                        const int64_t *cand_off, const int32_t *cand_idx, const uint16_t *q, const void *win_rows,
                        const uint8_t *win_scales, const void *pool_rows, const uint8_t *pool_scales,
                        const float *idx_q, const float *idx_w, int32_t idx_kdtype, const void *idx_k,
                        const uint8_t *idx_k_scales, const float *sink, int32_t *sel_io, float *out, float *lse) {
  size_t rb = (kv_dtype == ORC_KV_FP8) ? (size_t)d : (kv_dtype == ORC_KV_FP4) ? (size_t)d / 2 : 2 * (size_t)d;
  size_t sb = (kv_dtype == ORC_KV_FP8) ? (size_t)d / 32 : (kv_dtype == ORC_KV_FP4) ? (size_t)d / 16 : 0;
  const float *keys = NULL;
  float *dec = NULL;
  int32_t i;
  int err = ORC_OK;
  if (nq < 0 || !qs || pos0 < 0 || win_pos0 < 0 || win_pos0 > pos0 || n_win_rows < 0 || w < 0 || pool_len < 0)
    return ORC_EBADARG;
  if (mode < ORC_MODE_FULL || mode > ORC_MODE_WINDOW) return ORC_EBADARG;
  if (mode == ORC_MODE_REINDEX && (!cand_off || !cand_idx)) return ORC_EBADARG;
  if (idx_kdtype != ORC_IDXK_F32 && idx_kdtype != ORC_IDXK_MXFP4) return ORC_EBADARG;
  if ((mode == ORC_MODE_FULL || mode == ORC_MODE_REINDEX) && pool_len > 0) {
    if (!idx_k || !idx_q) return ORC_EBADARG;
    if (idx_kdtype == ORC_IDXK_F32) {
      keys = (const float *)idx_k;
    } else {
      int rc;
      if ((d_i % 32) != 0 || !idx_k_scales) return ORC_EBADARG;
      dec = (float *)malloc(sizeof(float) * (size_t)pool_len * (size_t)d_i);
      if (!dec) return ORC_ENOMEM;
      if ((rc = csa2o_dequant_mxfp4((const uint8_t *)idx_k, idx_k_scales, pool_len * d_i, dec)) != ORC_OK) {
        free(dec);
        return rc;
      }
      keys = dec;
    }
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (i = 0; i < nq; ++i) {
    const int64_t t = qs[i];
    const int64_t p = pos0 + t;
    int64_t lo = 0, cnt = 0;
    int32_t *sel = sel_io + (size_t)i * (size_t)k;
    int32_t nsel = k;
    int rc = csa2o_window_range(p, w, win_pos0, &lo, &cnt);
    if (rc == ORC_OK && (t < 0 || lo - win_pos0 + cnt > n_win_rows)) rc = ORC_EBADARG;
    if (rc == ORC_OK && (mode == ORC_MODE_FULL || mode == ORC_MODE_REINDEX)) {
      const int32_t *cl = (mode == ORC_MODE_REINDEX) ? cand_idx + cand_off[t] : NULL;
      const int64_t nc = (mode == ORC_MODE_REINDEX) ? cand_off[t + 1] - cand_off[t] : 0;
      int64_t r;
      if (pool_len == 0) { /* nothing to score: every slot is -1 */
        int32_t j;
        for (j = 0; j < k; ++j) sel[j] = -1;
        r = 0;
      } else {
        r = csa2o_select_query(mode, p, m, pool_len, h_i, d_i, idx_q + (size_t)t * (size_t)(h_i * d_i),
                               idx_w ? idx_w + (size_t)t * (size_t)h_i : NULL, relu, keys, cl, nc, k, sel, NULL);
      }
      if (r < 0) rc = (int)r;
    } else if (mode == ORC_MODE_WINDOW) {
      nsel = 0;
    }
    if (rc == ORC_OK)
      rc = csa2o_attend_query(h, d, kv_dtype, q + (size_t)t * (size_t)(h * d),
                              win_rows ? (const uint8_t *)win_rows + (size_t)(lo - win_pos0) * rb : NULL,
                              win_scales ? win_scales + (size_t)(lo - win_pos0) * sb : NULL, cnt, pool_rows,
                              pool_scales, pool_len, sel, nsel, sink, scale, out + (size_t)i * (size_t)(h * d),
                              lse ? lse + (size_t)i * (size_t)h : NULL);
    if (rc != ORC_OK) {
#pragma omp critical
      err = rc;
    }
  }
  free(dec);
  return err;
}
