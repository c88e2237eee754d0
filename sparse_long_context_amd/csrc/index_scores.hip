// Indexer scores (Reading Notes of DeepSeek-V4.1-Flash, section 3f C2 Step 2:
// sigma(j) = sum_h w_h * f(q^I_h . k^I_j) with the lightning-indexer form).
//
// Evaluation order is fixed so the selection that follows is reproducible bit
// for bit: per head, acc starts at +0 and takes fmaf(q[i], k[i], acc) for
// i = 0 .. 127 in order; then s = fmaf(w_h, f(acc_h), s) over heads in order;
// -0 becomes +0.  Heads are padded to a power of two with q = 0, w = 0, which
// leaves every sum unchanged (0 * finite adds an exact zero).
//
// Two kernels:
//  * decode: one workgroup per (query, 256 candidates).  The key rows are the
//    only large stream (512 B per candidate); they are staged through LDS in
//    four 32-float slabs with fully coalesced 128-byte row segments, the next
//    slab prefetched into registers while the current one is consumed.
//  * prefill: one sequence, many queries sharing the key rows, so the keys are
//    reused across queries: a register-tiled product of 128 queries x 128
//    candidates per workgroup (8 x 8 outputs per thread), each output's FMA
//    chain still running over i in order.
#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int kTile = 256;       // candidates per decode workgroup (one per thread)
constexpr int kSlab = 32;        // floats per staged key slab
constexpr int kSlabPad = 36;     // LDS row stride (floats): 16-byte aligned, conflict-free reads
constexpr int kSlabs = kIndexDim / kSlab;

__device__ __forceinline__ float finish_score(const float* acc, const float* w, int hp, int relu) {
  float s = 0.0f;
  for (int h = 0; h < hp; ++h) {
    float f = acc[h];
    if (relu) f = f > 0.0f ? f : 0.0f;
    s = __builtin_fmaf(w[h], f, s);
  }
  return s == 0.0f ? 0.0f : s;
}

template <int HP>
__global__ __launch_bounds__(kTile) void index_scores_decode(
    int32_t hi, int32_t relu, int32_t max_cand, const int64_t* __restrict__ pos,
    const int32_t* __restrict__ mode, const int32_t* __restrict__ ratio,
    const int64_t* __restrict__ pool_row0, const int32_t* __restrict__ pool_len,
    const int64_t* __restrict__ cand_off, const int32_t* __restrict__ cand_idx,
    const float* __restrict__ idx_q, const float* __restrict__ idx_w, const float* __restrict__ idx_k,
    float* __restrict__ scores, int64_t stride) {
  __shared__ float q_s[HP][kIndexDim];
  __shared__ float w_s[HP];
  __shared__ __attribute__((aligned(16))) float k_s[kTile][kSlabPad];
  __shared__ int64_t row_s[kTile];

  const int b = blockIdx.y;
  const int t = threadIdx.x;
  const int md = mode[b];
  if (md != CSA2_MODE_FULL && md != CSA2_MODE_REINDEX) return;
  const int64_t nv = n_valid_of(pos[b], ratio[b], md, pool_len[b]);
  int64_t n = (md == CSA2_MODE_FULL) ? nv : (cand_off[b + 1] - cand_off[b]);
  if (n > max_cand) n = max_cand;
  const int64_t j0 = (int64_t)blockIdx.x * kTile;
  if (j0 >= n) return;

  // query vectors and weights of this query (heads padded with zeros)
  for (int x = t; x < HP * kIndexDim; x += kTile) {
    const int h = x / kIndexDim, i = x % kIndexDim;
    q_s[h][i] = (h < hi) ? idx_q[((int64_t)b * hi + h) * kIndexDim + i] : 0.0f;
  }
  if (t < HP) w_s[t] = (t < hi) ? (idx_w ? idx_w[(int64_t)b * hi + t] : 1.0f) : 0.0f;

  // this thread's candidate: global key row, or -1 when it has none
  const int64_t j = j0 + t;
  int64_t row = -1;
  if (j < n) {
    int64_t r = (md == CSA2_MODE_FULL) ? j : (int64_t)cand_idx[cand_off[b] + j];
    if (r >= 0 && r < nv) row = pool_row0[b] + r;
  }
  row_s[t] = row;
  __syncthreads();

  // slab loader: 256 rows x 8 float4 pieces, 8 pieces per thread, 8 lanes per row
  float4 pf[8];
  auto fetch = [&](int s) {
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int p = it * kTile + t;
      const int c = p >> 3, part = p & 7;
      const int64_t r = row_s[c];
      pf[it] = (r >= 0) ? *reinterpret_cast<const float4*>(idx_k + r * kIndexDim + s * kSlab + part * 4)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int p = it * kTile + t;
      *reinterpret_cast<float4*>(&k_s[p >> 3][(p & 7) * 4]) = pf[it];
    }
  };

  float acc[HP];
#pragma unroll
  for (int h = 0; h < HP; ++h) acc[h] = 0.0f;

  fetch(0);
#pragma unroll 1
  for (int s = 0; s < kSlabs; ++s) {
    stash();
    __syncthreads();
    if (s + 1 < kSlabs) fetch(s + 1);
#pragma unroll
    for (int i4 = 0; i4 < kSlab / 4; ++i4) {
      const float4 k4 = *reinterpret_cast<const float4*>(&k_s[t][i4 * 4]);
      const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = s * kSlab + i4 * 4 + u;
#pragma unroll
        for (int h = 0; h < HP; ++h) acc[h] = __builtin_fmaf(q_s[h][i], kv[u], acc[h]);
      }
    }
    __syncthreads();
  }

  if (j < n) {
    float sc = -__builtin_inff();
    if (row >= 0) sc = finish_score(acc, w_s, HP, relu);
    scores[(int64_t)b * stride + j] = sc;
  }
}

// ---- prefill: queries x candidates, register tiled -------------------------
constexpr int kPQ = 128;  // queries per workgroup
constexpr int kPC = 128;  // candidates per workgroup
constexpr int kPK = 16;   // k slab

__global__ __launch_bounds__(256) void index_scores_prefill(
    int32_t T, const int64_t* __restrict__ pos, int32_t md, int32_t ratio, int32_t pool_len,
    const float* __restrict__ idx_q, const float* __restrict__ idx_w, int32_t relu,
    const float* __restrict__ idx_k, float* __restrict__ scores, int64_t stride) {
  __shared__ __attribute__((aligned(16))) float qs[kPK][kPQ];
  __shared__ __attribute__((aligned(16))) float ks[kPK][kPC];
  const int t = threadIdx.x;
  const int tq = t >> 4, tc = t & 15;
  const int q0 = blockIdx.y * kPQ, c0 = blockIdx.x * kPC;
  const int qlast = (q0 + kPQ < T ? q0 + kPQ : T) - 1;
  // the chunk's largest reachable count bounds every query's candidates here
  const int64_t nmax = n_valid_of(pos[qlast], ratio, md, pool_len);
  if (c0 >= nmax) return;

  float acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[a][c] = 0.0f;

  // loaders: 128 rows x 16 floats per slab = 512 float4, two per thread
  for (int s = 0; s < kIndexDim / kPK; ++s) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int p = it * 256 + t;
      const int r = p >> 2, part = p & 3;
      const int qq = q0 + r;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (qq < T) v = *reinterpret_cast<const float4*>(idx_q + (int64_t)qq * kIndexDim + s * kPK + part * 4);
      qs[part * 4 + 0][r] = v.x;
      qs[part * 4 + 1][r] = v.y;
      qs[part * 4 + 2][r] = v.z;
      qs[part * 4 + 3][r] = v.w;
      const int cc = c0 + r;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f);
      if (cc < nmax) kv = *reinterpret_cast<const float4*>(idx_k + (int64_t)cc * kIndexDim + s * kPK + part * 4);
      ks[part * 4 + 0][r] = kv.x;
      ks[part * 4 + 1][r] = kv.y;
      ks[part * 4 + 2][r] = kv.z;
      ks[part * 4 + 3][r] = kv.w;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPK; ++k) {
      const float4 qa = *reinterpret_cast<const float4*>(&qs[k][tq * 8]);
      const float4 qb = *reinterpret_cast<const float4*>(&qs[k][tq * 8 + 4]);
      const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
      float kv[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) kv[c] = ks[k][tc + 16 * c];
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[a][c] = __builtin_fmaf(qv[a], kv[c], acc[a][c]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int qq = q0 + tq * 8 + a;
    if (qq >= T) continue;
    const int64_t nq = n_valid_of(pos[qq], ratio, md, pool_len);
    const float wq = idx_w ? idx_w[qq] : 1.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int cc = c0 + tc + 16 * c;
      if (cc >= nq) continue;
      float f = acc[a][c];
      if (relu) f = f > 0.0f ? f : 0.0f;
      float s = __builtin_fmaf(wq, f, 0.0f);
      scores[(int64_t)qq * stride + cc] = (s == 0.0f) ? 0.0f : s;
    }
  }
}

}  // namespace

hipError_t launch_index_scores(const csa2_dims& d, int32_t B, const csa2_batch& bt, const float* idx_q,
                               const float* idx_w, const float* idx_k, float* scores, int64_t stride,
                               hipStream_t s) {
  if (B == 0 || bt.max_candidates == 0) return hipSuccess;
  dim3 grid((bt.max_candidates + kTile - 1) / kTile, B);
  const int hi = d.index_heads;
#define CSA2_IDX_ARGS                                                                                 \
  hi, d.index_relu, bt.max_candidates, bt.pos, bt.mode, bt.compress_ratio, bt.pool_row0, bt.pool_len, \
      bt.cand_off, bt.cand_idx, idx_q, idx_w, idx_k, scores, stride
  if (hi <= 1)
    hipLaunchKernelGGL(index_scores_decode<1>, grid, dim3(kTile), 0, s, CSA2_IDX_ARGS);
  else if (hi <= 4)
    hipLaunchKernelGGL(index_scores_decode<4>, grid, dim3(kTile), 0, s, CSA2_IDX_ARGS);
  else if (hi <= 16)
    hipLaunchKernelGGL(index_scores_decode<16>, grid, dim3(kTile), 0, s, CSA2_IDX_ARGS);
  else
    hipLaunchKernelGGL(index_scores_decode<64>, grid, dim3(kTile), 0, s, CSA2_IDX_ARGS);
#undef CSA2_IDX_ARGS
  return hipGetLastError();
}

hipError_t launch_index_scores_prefill(const csa2_dims& d, int32_t T, const int64_t* pos, int32_t mode,
                                       int32_t ratio, int32_t pool_len, const float* idx_q,
                                       const float* idx_w, const float* idx_k, float* scores,
                                       int64_t stride, hipStream_t s) {
  if (T == 0 || pool_len == 0) return hipSuccess;
  dim3 grid((pool_len + kPC - 1) / kPC, (T + kPQ - 1) / kPQ);
  hipLaunchKernelGGL(index_scores_prefill, grid, dim3(256), 0, s, T, pos, mode, ratio, pool_len, idx_q,
                     idx_w, d.index_relu, idx_k, scores, stride);
  return hipGetLastError();
}

}  // namespace csa2
