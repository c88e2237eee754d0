// The steps on either side of the attention: the compressor that writes the
// compressed KV cache, and the de-rotation of the attention output.
//
// Compressor (Reading Notes of DeepSeek-V4.1-Flash, section 3f C2 Step 1: a
// block of m consecutive tokens becomes one entry, sum_u softmax_u(g_u) (.) c_u
// with the softmax over the block's tokens taken per channel; PocketLLM
// "DeepSeek-V4.1-Flash", "The compressor": pooled in fp32, then RMS-normed, no
// gate at ratio 1).  One workgroup per group; fp32 throughout.
//
// The compressor's decode step (section 3f C2 Step 1: entry j exists once its
// m tokens are in; PocketLLM "DeepSeek-V4.1-Flash", "The CSA2 attention
// layers": the trailing partial group waits in state between calls, and a step
// that closes no group emits nothing).
//
// De-rotation ("DeepSeek-V4.1-Flash on WASTE", What is new, 1. CSA2: the rope
// dims of the attention output are rotated by the conjugate of the query's
// rotation).  Pair i of the rope dims turns by -pos * inv_freq[i]; the angle,
// its sine and cosine are taken in fp64 (pos * freq reaches 10^6 radians,
// where fp32 would lose the angle) and rounded to fp32 for the fp32 turn.
#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int kCThreads = 256;

// One group's latent: the thread's channels i = t, t + 256, .. pooled over the
// group's m rows (row u from cj / gj, except row un, which comes from cn / gn:
// the token a decode step brings), then RMS-normed over the d channels by the
// whole workgroup.  Every workgroup thread must call it.
__device__ __forceinline__ void compress_group(int32_t m, int32_t d, const float* cj, const float* gj, int un,
                                               const float* cn, const float* gn, const float* w, float eps,
                                               float* outj, float* red_s) {
  const int t = threadIdx.x;
  float ss = 0.0f;
  // each thread pools its channels (at most kMaxCompressDim / kCThreads of them)
  float pooled[kMaxCompressDim / kCThreads];
#pragma unroll
  for (int k = 0; k < kMaxCompressDim / kCThreads; ++k) {
    const int i = t + k * kCThreads;
    float v = 0.0f;
    if (i < d) {
      if (m == 1) {
        v = (un == 0 ? cn : cj)[i];
      } else {
        float mx = -__builtin_inff();
        for (int u = 0; u < m; ++u) mx = fmaxf(mx, u == un ? gn[i] : gj[(int64_t)u * d + i]);
        float z = 0.0f, acc = 0.0f;
        for (int u = 0; u < m; ++u) {
          const float e = __expf((u == un ? gn[i] : gj[(int64_t)u * d + i]) - mx);
          z += e;
          acc = __builtin_fmaf(e, u == un ? cn[i] : cj[(int64_t)u * d + i], acc);
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
    if (i < d) outj[i] = pooled[k] * r * w[i];
  }
}

__global__ __launch_bounds__(kCThreads) void compress_kernel(int32_t m, int32_t d, const float* __restrict__ c,
                                                             const float* __restrict__ g,
                                                             const float* __restrict__ w, float eps,
                                                             float* __restrict__ out) {
  __shared__ float red_s[kCThreads / 64];
  const int64_t j = blockIdx.x;
  compress_group(m, d, c + j * (int64_t)m * d, g ? g + j * (int64_t)m * d : nullptr, -1, nullptr, nullptr, w, eps,
                 out + j * d, red_s);
}

// Decode step: one workgroup per sequence.  The new token goes to its slot of
// the sequence's partial-group state; the step that fills the last slot pools
// the group, reading the new token from its input rather than back from the
// state, so the latent equals compress_kernel's over the same group.
__global__ __launch_bounds__(kCThreads) void compress_step_kernel(int32_t m, int32_t d,
                                                                  const int64_t* __restrict__ pos,
                                                                  const float* __restrict__ c_new,
                                                                  const float* __restrict__ g_new, float* kv_state,
                                                                  float* score_state, const float* __restrict__ w,
                                                                  float eps, float* __restrict__ out,
                                                                  int32_t* __restrict__ emit_idx) {
  __shared__ float red_s[kCThreads / 64];
  const int b = blockIdx.x, t = threadIdx.x;
  const int64_t p = pos[b];
  if (p < 0) {  // no slot: nothing written, nothing emitted
    if (t == 0) emit_idx[b] = -1;
    return;
  }
  const float* cn = c_new + (int64_t)b * d;
  const int u = (int)(p % m);
  const bool closes = u == m - 1;
  if (t == 0) emit_idx[b] = closes ? (int32_t)((p + 1) / m - 1) : -1;
  if (m == 1) {
    compress_group(1, d, nullptr, nullptr, 0, cn, nullptr, w, eps, out + (int64_t)b * d, red_s);
    return;
  }
  const float* gn = g_new + (int64_t)b * d;
  float* cs = kv_state + (int64_t)b * m * d;
  float* gs = score_state + (int64_t)b * m * d;
  for (int i = t; i < d; i += kCThreads) {
    cs[(int64_t)u * d + i] = cn[i];
    gs[(int64_t)u * d + i] = gn[i];
  }
  if (closes) compress_group(m, d, cs, gs, u, cn, gn, w, eps, out + (int64_t)b * d, red_s);
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

hipError_t launch_compress_step(int32_t B, int32_t m, int32_t d, const int64_t* pos, const float* c_new,
                                const float* g_new, float* kv_state, float* score_state, const float* w, float eps,
                                float* out, int32_t* emit_idx, hipStream_t s) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(compress_step_kernel, dim3((unsigned)B), dim3(kCThreads), 0, s, m, d, pos, c_new, g_new,
                     kv_state, score_state, w, eps, out, emit_idx);
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
