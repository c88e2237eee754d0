// Top-K selection (Reading Notes of DeepSeek-V4.1-Flash, section 3f C2 Step 2:
// keep the K best-scoring entries; PocketLLM "DeepSeek-V4.1-Flash",
// "Correctness and precision": unused slots hold -1).
//
// Order: score descending, then row ascending (the lowest row wins a tie); +0
// and -0 tie.  Output: the chosen rows in ascending order, then -1s.
//
// One workgroup (1024 threads, 16 waves) per query:
//  1. scores map to order-preserving 32-bit keys (ineligible slots -> key 0,
//     below every finite score and -inf), kept in LDS when they fit;
//  2. a 4-pass 8-bit radix select finds the key T of the K-th best and how
//     many of the candidates equal to T are taken (the lowest-row ones);
//  3. one ordered pass over the candidates, with wave ballots and a cross-wave
//     prefix, writes the selected rows in ascending order.
#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kLdsKeys = 16384;  // keys cached in LDS (64 KiB); larger queries re-read scores

__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;  // -0 ties with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kThreads) void topk_kernel(
    int32_t K, int32_t max_cand, const int64_t* __restrict__ pos, const int32_t* __restrict__ mode,
    const int32_t* __restrict__ ratio, const int32_t* __restrict__ pool_len,
    const int64_t* __restrict__ cand_off, const int32_t* __restrict__ cand_idx,
    const float* __restrict__ scores, int64_t stride, int32_t* __restrict__ topk_idx) {
  __shared__ uint32_t keys_s[kLdsKeys];
  __shared__ uint32_t hist_s[kWaves][256];
  __shared__ uint32_t wcnt_s[2][kWaves];
  __shared__ uint32_t sel_s[4];  // chosen digit, count above it
  __shared__ uint32_t elig_s;

  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const int md = mode[b];
  if (md != CSA2_MODE_FULL && md != CSA2_MODE_REINDEX) return;
  const int64_t nv = n_valid_of(pos[b], ratio[b], md, pool_len[b]);
  int64_t n64 = (md == CSA2_MODE_FULL) ? nv : (cand_off[b + 1] - cand_off[b]);
  if (n64 > max_cand) n64 = max_cand;
  const int n = (int)n64;
  const int32_t* lst = (md == CSA2_MODE_REINDEX) ? cand_idx + cand_off[b] : nullptr;
  const float* sc = scores + (int64_t)b * stride;
  const bool in_lds = n <= kLdsKeys;

  auto row_of = [&](int i) -> int32_t { return lst ? lst[i] : i; };
  auto eligible = [&](int i) -> bool {
    const int32_t r = row_of(i);
    return r >= 0 && r < nv;
  };
  auto key_at = [&](int i) -> uint32_t {
    if (in_lds) return keys_s[i];
    return eligible(i) ? order_key(sc[i]) : 0u;
  };

  if (t == 0) elig_s = 0;
  __syncthreads();
  uint32_t my_elig = 0;
  for (int i = t; i < n; i += kThreads) {
    const bool e = eligible(i);
    my_elig += e;
    if (in_lds) keys_s[i] = e ? order_key(sc[i]) : 0u;
  }
  // eligible count
  for (int o = 32; o > 0; o >>= 1) my_elig += __shfl_xor(my_elig, o);
  if (lane == 0) atomicAdd(&elig_s, my_elig);
  __syncthreads();
  const uint32_t n_elig = elig_s;

  uint32_t thr = 0;           // key of the K-th best
  uint32_t take_eq = 0;       // how many keys equal to thr are taken
  bool take_all = n_elig <= (uint32_t)K;
  if (!take_all) {
    uint32_t prefix = 0, pmask = 0, krem = (uint32_t)K;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int x = t; x < kWaves * 256; x += kThreads) (&hist_s[0][0])[x] = 0;
      __syncthreads();
      for (int i = t; i < n; i += kThreads) {
        const uint32_t k = key_at(i);
        if ((k & pmask) == prefix) atomicAdd(&hist_s[wv][(k >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (wv == 0) {
        // lane owns digits 4*lane .. 4*lane+3; total them over the waves
        uint32_t c[4], tot = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          uint32_t a = 0;
          for (int w = 0; w < kWaves; ++w) a += hist_s[w][4 * lane + u];
          c[u] = a;
          tot += a;
        }
        // count of keys in digits owned by higher lanes (exclusive suffix sum)
        uint32_t suf = tot;
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t v = __shfl_down(suf, o);
          if (lane + o < 64) suf += v;
        }
        uint32_t above = suf - tot;
#pragma unroll
        for (int u = 3; u >= 0; --u) {
          if (above < krem && krem <= above + c[u]) {
            sel_s[0] = 4 * lane + u;
            sel_s[1] = above;
          }
          above += c[u];
        }
      }
      __syncthreads();
      const uint32_t dg = sel_s[0];
      krem -= sel_s[1];
      prefix |= dg << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    thr = prefix;
    take_eq = krem;
  }

  // ordered compaction: candidate i goes to slot (number selected before it)
  int32_t* out = topk_idx + (int64_t)b * K;
  uint32_t base_sel = 0, base_eq = 0;
  for (int i0 = 0; i0 < n; i0 += kThreads) {
    const int i = i0 + t;
    bool gt = false, eq = false;
    if (i < n) {
      if (take_all) {
        gt = eligible(i);
      } else {
        const uint32_t k = key_at(i);
        gt = k > thr;
        eq = k == thr;
      }
    }
    const uint64_t meq = __ballot(eq);
    if (lane == 0) wcnt_s[0][wv] = __popcll(meq);
    __syncthreads();
    uint32_t eq_before = base_eq, eq_tot = 0;
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t c = wcnt_s[0][w];
      if (w < wv) eq_before += c;
      eq_tot += c;
    }
    eq_before += __popcll(meq & ((1ull << lane) - 1ull));
    const bool take = gt || (eq && eq_before < take_eq);
    const uint64_t msel = __ballot(take);
    if (lane == 0) wcnt_s[1][wv] = __popcll(msel);
    __syncthreads();
    uint32_t sel_before = base_sel, sel_tot = 0;
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t c = wcnt_s[1][w];
      if (w < wv) sel_before += c;
      sel_tot += c;
    }
    sel_before += __popcll(msel & ((1ull << lane) - 1ull));
    if (take && sel_before < (uint32_t)K) out[sel_before] = row_of(i);
    base_eq += eq_tot;
    base_sel += sel_tot;
    __syncthreads();
  }
  for (int x = (int)(base_sel < (uint32_t)K ? base_sel : K) + t; x < K; x += kThreads) out[x] = -1;
}

}  // namespace

hipError_t launch_topk(const csa2_dims& d, int32_t B, const csa2_batch& bt, const float* scores,
                       int64_t stride, int32_t* topk_idx, hipStream_t s) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(B), dim3(kThreads), 0, s, d.index_topk, bt.max_candidates, bt.pos,
                     bt.mode, bt.compress_ratio, bt.pool_len, bt.cand_off, bt.cand_idx, scores, stride,
                     topk_idx);
  return hipGetLastError();
}

}  // namespace csa2
