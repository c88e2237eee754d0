// The cache writer's FP4 quantizers (Reading Notes of DeepSeek-V4.1-Flash,
// section 3f C4: 4-bit E2M1 codes times a scale shared by a block, s = amax/6,
// code = round_E2M1(x / s); PocketLLM "DeepSeek-V4.1-Flash", "The CSA2
// attention layers": compressed KV in FP4 with an E4M3 scale per 16 values,
// indexer keys in FP4 with an E8M0 scale per 32, the E4M3 scale being
// e4m3(amax / 6) with amax floored at 6 * 2^-9 and the E8M0 scale
// 2^round(log2(amax / 6)); FP4 ties round to the even code).
//
// One thread per scale block; both are plain elementwise passes over fp32 rows.
#include "csa2_internal.h"

namespace csa2 {
namespace {

// Nearest E2M1 magnitude code of a >= 0 (0, .5, 1, 1.5, 2, 3, 4, 6), ties to
// the even code, saturating at 6: one step per midpoint, a tie staying below
// when the lower code is even (0, 1, 2 -> 1.25, 2.5, 5) and moving up when
// the upper one is (0.75, 1.75, 3.5).
__device__ __forceinline__ uint32_t e2m1_mag(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
         (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
}

__device__ __forceinline__ uint32_t e2m1_code(float q) {
  const uint32_t m = e2m1_mag(fabsf(q));
  return (q < 0.0f && m != 0u) ? (m | 8u) : m;
}

// fp32 (finite, > 0) -> FP8 E4M3 ("fn": bias 7, max 448), nearest-even,
// saturating at 448.  Integer rounding of the fp32 bit pattern.
__device__ __forceinline__ uint32_t f32_to_e4m3_pos(float a) {
  if (a >= 448.0f) return 0x7Eu;
  if (a < 0.015625f) {  // below 2^-6: subnormal quantum 2^-9
    const uint32_t m = (uint32_t)__builtin_rintf(a * 512.0f);  // exact scaling, nearest-even
    return m;  // m == 8 is 2^-6, the first normal (exponent field 1, mantissa 0)
  }
  const uint32_t bits = __float_as_uint(a);
  uint32_t q = bits >> 20;  // exponent and top 3 mantissa bits
  const uint32_t r = bits & 0xFFFFFu, half = 0x80000u;
  if (r > half || (r == half && (q & 1u))) ++q;  // may carry into the exponent
  const uint32_t e = (q >> 3) - 127u + 7u, m = q & 7u;
  if (e > 15u || (e == 15u && m == 7u)) return 0x7Eu;
  return (e << 3) | m;
}

__device__ __forceinline__ float e4m3_pos_value(uint32_t byte) {
  const uint32_t e = byte >> 3, m = byte & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

__global__ __launch_bounds__(256) void quantize_fp4_kv_kernel(int64_t nblk, const float* __restrict__ src,
                                                              uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales) {
  const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (blk >= nblk) return;
  float x[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 v = *reinterpret_cast<const float4*>(src + blk * 16 + 4 * i);
    x[4 * i] = v.x, x[4 * i + 1] = v.y, x[4 * i + 2] = v.z, x[4 * i + 3] = v.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = fmaxf(amax, 6.0f * 0.001953125f);
  const uint32_t sb = f32_to_e4m3_pos(__fdiv_rn(amax, 6.0f));
  const float s = e4m3_pos_value(sb);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) lo |= e2m1_code(__fdiv_rn(x[i], s)) << (4 * i);
#pragma unroll
  for (int i = 0; i < 8; ++i) hi |= e2m1_code(__fdiv_rn(x[8 + i], s)) << (4 * i);
  *reinterpret_cast<uint2*>(codes + blk * 8) = make_uint2(lo, hi);
  scales[blk] = (uint8_t)sb;
}

__global__ __launch_bounds__(256) void quantize_mxfp4_kernel(int64_t nblk, const float* __restrict__ src,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (blk >= nblk) return;
  float x[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 v = *reinterpret_cast<const float4*>(src + blk * 32 + 4 * i);
    x[4 * i] = v.x, x[4 * i + 1] = v.y, x[4 * i + 2] = v.z, x[4 * i + 3] = v.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const float y = __fdiv_rn(amax, 6.0f);
  int e = -126;
  if (y > 0.0f) {
    int k;
    const float f = frexpf(y, &k);  // y = f 2^k, f in [0.5, 1): y = (2f) 2^(k-1)
    // log2 rounds up exactly when 2f > sqrt 2; the largest fp32 below sqrt 2
    // is 1.41421353816986083984375, so 2f > sqrt 2 iff 2f exceeds it
    e = (k - 1) + ((2.0f * f > 1.41421353816986083984375f) ? 1 : 0);
  }
  e = e < -126 ? -126 : (e > 127 ? 127 : e);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) w[i / 8] |= e2m1_code(ldexpf(x[i], -e)) << (4 * (i % 8));
  *reinterpret_cast<uint4*>(codes + blk * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  scales[blk] = (uint8_t)(e + 127);
}

}  // namespace

hipError_t launch_quantize_fp4_kv(int64_t n_rows, int32_t d, const float* src, uint8_t* codes, uint8_t* scales,
                                  hipStream_t s) {
  const int64_t nblk = n_rows * (d / 16);
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_fp4_kv_kernel, dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, s, nblk, src, codes,
                     scales);
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp4(int64_t n_rows, int32_t d, const float* src, uint8_t* codes, uint8_t* scales,
                                 hipStream_t s) {
  const int64_t nblk = n_rows * (d / 32);
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_mxfp4_kernel, dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, s, nblk, src, codes,
                     scales);
  return hipGetLastError();
}

}  // namespace csa2
