/*
 * csa2_synth.c -- seeded synthetic inputs for the CSA2 attention step.
 *
 * This module only draws numbers and stores them in the input formats; it
 * holds none of the attention's arithmetic.  It is the one piece shared by the
 * HIP path's tests/benchmark and the CPU oracle, which both read the bytes it
 * writes.
 *
 * Generator (counter-based, so any slice can be regenerated on its own and the
 * result does not depend on the thread count):
 *   key(seed, stream) = mix(mix(seed) ^ (stream * 0xD1B54A32D192ED03))
 *   U(c)   = ((mix(key + (c + 1) * 0x9E3779B97F4A7C15) >> 11) + 1) * 2^-53,  in (0, 1]
 *   mix    = the SplitMix64 output function (Steele, Lea and Flood, OOPSLA 2014):
 *            z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
 *            z *= 0x94D049BB133111EB; z ^= z >> 31
 *   N(i)   = Box-Muller on the pair p = i / 2:
 *            r = sqrt(-2 ln U(2p)), t = 2 pi U(2p+1); N = r cos t (even i), r sin t (odd i)
 * Storage: the double value times its scale is rounded to fp32 (nearest-even);
 * bf16 tensors round that fp32 value to bf16 (nearest-even).  FP8 tensors are
 * E4M3 ("fn": bias 7, max 448) codes with one UE8M0 scale per 32 consecutive
 * values: the scale is the smallest power of two 2^e with amax <= 448 * 2^e
 * (e = 0 for an all-zero block), each code is the nearest-even E4M3 value of
 * x / 2^e, and the stored scale byte is e + 127.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBULL;
  z ^= z >> 31;
  return z;
}

static uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed) ^ (stream * 0xD1B54A32D192ED03ULL));
}

static uint64_t draw_u64(uint64_t key, uint64_t c) {
  return mix64(key + (c + 1) * 0x9E3779B97F4A7C15ULL);
}

static double draw_unit(uint64_t key, uint64_t c) {
  return (double)((draw_u64(key, c) >> 11) + 1) * ldexp(1.0, -53);
}

static double draw_normal(uint64_t key, uint64_t i) {
  uint64_t p = i >> 1;
  double r = sqrt(-2.0 * log(draw_unit(key, 2 * p)));
  double t = 2.0 * M_PI * draw_unit(key, 2 * p + 1);
  return (i & 1) ? r * sin(t) : r * cos(t);
}

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Nearest-even E4M3 code of |a| <= 448 (sign handled by the caller). */
static uint8_t e4m3_code_abs(double a) {
  if (a < ldexp(1.0, -6)) { /* subnormal range: step 2^-9 */
    double m = nearbyint(ldexp(a, 9));
    return (uint8_t)m; /* m == 8 is exactly the smallest normal, code 0x08 */
  } else {
    int x, e;
    double f = frexp(a, &x), m;
    (void)f;
    e = x - 1; /* a in [2^e, 2^(e+1)) */
    m = nearbyint((ldexp(a, -e) - 1.0) * 8.0);
    if (m == 8.0) {
      m = 0.0;
      e += 1;
    }
    return (uint8_t)(((e + 7) << 3) | (int)m);
  }
}

/* out[j] = bf16(fp32(N(start + j) * scale)) */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t start, uint64_t count, double scale,
                       uint16_t *out) {
  uint64_t key = stream_key(seed, stream);
  int64_t j;
#pragma omp parallel for schedule(static)
  for (j = 0; j < (int64_t)count; ++j)
    out[j] = f32_to_bf16_rne((float)(draw_normal(key, start + (uint64_t)j) * scale));
}

/* out[j] = fp32(N(start + j) * scale) */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t start, uint64_t count, double scale,
                      float *out) {
  uint64_t key = stream_key(seed, stream);
  int64_t j;
#pragma omp parallel for schedule(static)
  for (j = 0; j < (int64_t)count; ++j) out[j] = (float)(draw_normal(key, start + (uint64_t)j) * scale);
}

/* Rows of d values (d a multiple of 32) quantized to E4M3 + UE8M0 per 32.
 * Value index of row r, column c is (start_row + r) * d + c. */
int synth_normal_fp8(uint64_t seed, uint64_t stream, uint64_t start_row, uint64_t rows, int d,
                     double scale, uint8_t *codes, uint8_t *scales) {
  uint64_t key = stream_key(seed, stream);
  int64_t r;
  int bad = 0;
  if (d <= 0 || d % 32) return -1;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (r = 0; r < (int64_t)rows; ++r) {
    float x[32];
    int blk, c;
    for (blk = 0; blk < d / 32; ++blk) {
      double amax = 0.0;
      int e = 0;
      for (c = 0; c < 32; ++c) {
        uint64_t i = (start_row + (uint64_t)r) * (uint64_t)d + (uint64_t)(blk * 32 + c);
        x[c] = (float)(draw_normal(key, i) * scale);
        if (fabs((double)x[c]) > amax) amax = fabs((double)x[c]);
      }
      if (amax > 0.0) {
        int xx;
        frexp(amax / 448.0, &xx);
        e = xx;
        while (amax > ldexp(448.0, e)) ++e;
        while (amax <= ldexp(448.0, e - 1)) --e;
      }
      if (e + 127 < 0 || e + 127 > 254) bad = 1;
      scales[(size_t)r * (size_t)(d / 32) + (size_t)blk] = (uint8_t)(e + 127);
      for (c = 0; c < 32; ++c) {
        double v = ldexp((double)x[c], -e);
        uint8_t code = e4m3_code_abs(fabs(v));
        if (v < 0.0 || (v == 0.0 && signbit(v))) code |= 0x80;
        codes[(size_t)r * (size_t)d + (size_t)(blk * 32 + c)] = code;
      }
    }
  }
  return bad ? -2 : 0;
}

/* Uniform integers lo + (U64(start + j) mod (hi - lo + 1)); the modulo bias is
 * below 2^-40 for the ranges used here. */
void synth_uniform_int(uint64_t seed, uint64_t stream, uint64_t start, uint64_t count, int64_t lo,
                       int64_t hi, int64_t *out) {
  uint64_t key = stream_key(seed, stream), span = (uint64_t)(hi - lo) + 1;
  uint64_t j;
  for (j = 0; j < count; ++j) out[j] = lo + (int64_t)(draw_u64(key, start + j) % span);
}

static int cmp_i32(const void *a, const void *b) {
  int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x > y) - (x < y);
}

/* k distinct integers drawn uniformly from [0, n) by a partial Fisher-Yates
 * shuffle driven by U64 draws, returned in ascending order (all of [0, n)
 * when k >= n).  Returns the number written. */
int64_t synth_sample_distinct(uint64_t seed, uint64_t stream, int64_t n, int64_t k, int32_t *out) {
  uint64_t key = stream_key(seed, stream);
  int32_t *perm;
  int64_t i, take = k < n ? k : n;
  if (n <= 0 || take <= 0) return 0;
  perm = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
  if (!perm) return -1;
  for (i = 0; i < n; ++i) perm[i] = (int32_t)i;
  for (i = 0; i < take; ++i) {
    int64_t j = i + (int64_t)(draw_u64(key, (uint64_t)i) % (uint64_t)(n - i));
    int32_t t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
  memcpy(out, perm, sizeof(int32_t) * (size_t)take);
  free(perm);
  qsort(out, (size_t)take, sizeof(int32_t), cmp_i32);
  return take;
}
