// The steps on either side of the attention: the compressor that writes the
// compressed KV cache, and the de-rotation of the attention output.
//
// Compressor (Reading Notes of DeepSeek-V4.1-Flash, section 3f C2 Step 1: a
// block of m consecutive tokens becomes one entry, sum_u softmax_u(g_u) (.) c_u
// with the softmax over the block's tokens taken per channel; PocketLLM
// "DeepSeek-V4.1-Flash", "The compressor": pooled in fp32, then RMS-normed, no
// gate at ratio 1).  One workgroup per group; fp32 throughout.
//
// De-rotation ("DeepSeek-V4.1-Flash on WASTE", What is new, 1. CSA2: the rope
// dims of the attention output are rotated by the conjugate of the query's
// rotation).  Pair i of the rope dims turns by -pos * inv_freq[i]; the angle,
// its sine and cosine and the rotation are taken in fp64, since pos * freq
// reaches 10^6 radians where fp32 would lose the angle.
#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int kCThreads = 256;

__global__ __launch_bounds__(kCThreads) void compress_kernel(int32_t m, int32_t d, const float* __restrict__ c,
                                                             const float* __restrict__ g,
                                                             const float* __restrict__ w, float eps,
                                                             float* __restrict__ out) {
  __shared__ float red_s[kCThreads / 64];
  const int64_t j = blockIdx.x;
  const int t = threadIdx.x;
  const float* cj = c + j * (int64_t)m * d;
  const float* gj = g ? g + j * (int64_t)m * d : nullptr;
  float ss = 0.0f;
  // each thread pools its channels (at most kMaxCompressDim / kCThreads of them)
  float pooled[kMaxCompressDim / kCThreads];
#pragma unroll
  for (int k = 0; k < kMaxCompressDim / kCThreads; ++k) {
    const int i = t + k * kCThreads;
    float v = 0.0f;
    if (i < d) {
      if (m == 1) {
        v = cj[i];
      } else {
        float mx = -__builtin_inff();
        for (int u = 0; u < m; ++u) mx = fmaxf(mx, gj[(int64_t)u * d + i]);
        float z = 0.0f, acc = 0.0f;
        for (int u = 0; u < m; ++u) {
          const float e = __expf(gj[(int64_t)u * d + i] - mx);
          z += e;
          acc = __builtin_fmaf(e, cj[(int64_t)u * d + i], acc);
        }
        v = acc / z;
      }
      ss = __builtin_fmaf(v, v, ss);
    }
    pooled[k] = v;
  }
  // sum of squares over the workgroup
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((t & 63) == 0) red_s[t >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int k = 0; k < kCThreads / 64; ++k) tot += red_s[k];
  const float r = 1.0f / sqrtf(tot / (float)d + eps);
#pragma unroll
  for (int k = 0; k < kMaxCompressDim / kCThreads; ++k) {
    const int i = t + k * kCThreads;
    if (i < d) out[j * d + i] = pooled[k] * r * w[i];
  }
}

__global__ __launch_bounds__(256) void derotate_kernel(const int64_t* __restrict__ pos, int32_t rope_off,
                                                       int32_t rope_dims, const double* __restrict__ inv_freq,
                                                       float* __restrict__ out) {
  __shared__ float cs_s[kMaxRopeDims / 2], sn_s[kMaxRopeDims / 2];
  const int b = blockIdx.x, t = threadIdx.x;
  const int np = rope_dims / 2;
  if (t < np) rope_angle(pos[b], inv_freq[t], cs_s[t], sn_s[t]);
  __syncthreads();
  float* ob = out + (int64_t)b * kHeads * kDim;
  for (int x = t; x < kHeads * np; x += 256) {
    const int h = x / np, i = x % np;
    float* p = ob + (int64_t)h * kDim + rope_off + 2 * i;
    rope_turn(p[0], p[1], cs_s[i], sn_s[i]);
  }
}

// one thread per (query, pair): the cosine and sine the fused epilogues turn by
__global__ __launch_bounds__(256) void rope_table_kernel(int32_t B, const int64_t* __restrict__ pos, RopeOut r,
                                                         float2* __restrict__ table) {
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t b = x / kRopePairs;
  const int i = (int)(x % kRopePairs);
  if (b >= B || 2 * i >= r.dims) return;
  float c, s;
  rope_angle(pos[b], r.inv_freq[i], c, s);
  table[x] = make_float2(c, s);
}

}  // namespace

size_t rope_table_bytes(int32_t B) { return (size_t)(B > 0 ? B : 0) * kRopePairs * sizeof(float2); }

hipError_t launch_rope_table(int32_t B, const int64_t* pos, const RopeOut& r, hipStream_t s) {
  if (B <= 0 || r.inv_freq == nullptr || r.table == nullptr) return hipSuccess;
  const int64_t n = (int64_t)B * kRopePairs;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, B, pos, r,
                     const_cast<float2*>(r.table));
  return hipGetLastError();
}

hipError_t launch_compress(int64_t n_groups, int32_t m, int32_t d, const float* c, const float* g, const float* w,
                           float eps, float* out, hipStream_t s) {
  if (n_groups == 0) return hipSuccess;
  hipLaunchKernelGGL(compress_kernel, dim3((unsigned)n_groups), dim3(kCThreads), 0, s, m, d, c, m > 1 ? g : nullptr,
                     w, eps, out);
  return hipGetLastError();
}

hipError_t launch_derotate(int32_t B, const int64_t* pos, int32_t rope_off, int32_t rope_dims,
                           const double* inv_freq, float* out, hipStream_t s) {
  if (B == 0 || rope_dims == 0) return hipSuccess;
  hipLaunchKernelGGL(derotate_kernel, dim3(B), dim3(256), 0, s, pos, rope_off, rope_dims, inv_freq, out);
  return hipGetLastError();
}

}  // namespace csa2
