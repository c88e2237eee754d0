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
//  * decode: one workgroup per (query, 32 candidates).  The key rows are the
//    only large stream (512 B per candidate); 256 threads load them with
//    coalesced 16-byte loads into LDS, then each of 32 lanes runs one
//    candidate's FMA chain out of LDS.
//  * decode with MXFP4 keys (E2M1 codes + one E8M0 scale per 32, 68 B per
//    candidate; PocketLLM "DeepSeek-V4.1-Flash", "The CSA2 attention layers"):
//    one workgroup (one wave) per (query, 64 candidates); the code rows come in with
//    coalesced 16-byte loads through LDS, and each thread widens its own row to
//    fp32 exactly and runs its FMA chain, so the score is the one fp32 keys
//    holding the decoded values would give.
//  * prefill: one sequence, many queries sharing the key rows, so the keys are
//    reused across queries: a register-tiled product of 128 queries x 128
//    candidates per workgroup (8 x 8 outputs per thread), each output's FMA
//    chain still running over i in order.
#include "csa2_internal.h"

namespace csa2 {
namespace {


__device__ __forceinline__ float finish_score(const float* acc, const float* w, int hp, int relu) {
  float s = 0.0f;
  for (int h = 0; h < hp; ++h) {
    float f = acc[h];
    if (relu) f = f > 0.0f ? f : 0.0f;
    s = __builtin_fmaf(w[h], f, s);
  }
  return s == 0.0f ? 0.0f : s;
}

// 256 threads move the 32 key rows of a workgroup (16 KiB, contiguous for
// FULL queries) with plain coalesced 16-byte loads, four per thread, into an
// XOR-swizzled LDS tile; then 32 lanes each run one candidate's FMA chain out
// of LDS.  Tiny workgroups keep many loads in flight per CU, which is what
// reaches the HBM read ceiling here.
constexpr int kRows = 32;                          // candidates per workgroup
constexpr int kThreads = 256;
constexpr int kUnits = kIndexDim / 4;              // 32 units of 16 B per key row
constexpr int kPieces = kRows * kUnits / kThreads; // 4 loads per thread

__device__ __forceinline__ int key_unit_swz(int r, int u) { return u ^ (r & 15); }

// Index keys are read once per step and the stream is larger than the last
// level cache, so their loads carry the non-temporal hint: streaming reads
// with it reach about 7.2 TB/s here against 6.4 TB/s without.
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream(const float* p) {
  const f32x4v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint4 load_stream(const uint8_t* p) {
  const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// With one or a few index heads: eight waves per SIMD (at most 64 VGPRs), so
// eight workgroups per CU keep 128 KiB of key rows in flight, where the
// register use the compiler picks by itself (80) allows six.
template <int HP>
__global__ __launch_bounds__(kThreads, HP <= 4 ? 8 : 1) void index_scores_decode(
    int32_t hi, int32_t relu, int32_t max_cand, const int64_t* __restrict__ pos,
    const int32_t* __restrict__ mode, const int32_t* __restrict__ ratio,
    const int64_t* __restrict__ pool_row0, const int32_t* __restrict__ pool_len,
    const int64_t* __restrict__ cand_off, const int32_t* __restrict__ cand_idx,
    const float* __restrict__ idx_q, const float* __restrict__ idx_w, const float* __restrict__ idx_k,
    float* __restrict__ scores, int64_t stride) {
  __shared__ __attribute__((aligned(16))) float k_s[kRows * kIndexDim];
  __shared__ __attribute__((aligned(16))) float q_s[HP][kIndexDim];
  __shared__ float w_s[HP];
  __shared__ int64_t row_s[kRows];

  const int b = blockIdx.y;
  const int t = threadIdx.x;
  const int md = mode[b];
  if (md != CSA2_MODE_FULL && md != CSA2_MODE_REINDEX) return;
  const int64_t nv = n_valid_of(pos[b], ratio[b], md, pool_len[b]);
  // a REINDEX query without lists (cand_off NULL) has an empty list
  int64_t n = (md == CSA2_MODE_FULL) ? nv : (cand_off ? cand_off[b + 1] - cand_off[b] : 0);
  if (n > max_cand) n = max_cand;
  const int64_t j0 = (int64_t)blockIdx.x * kRows;
  if (j0 >= n) return;

  if (t < kRows) {  // candidate rows (pool-relative), -1 when there is none
    const int64_t j = j0 + t;
    int64_t r = -1;
    if (j < n) {
      const int64_t rr = (md == CSA2_MODE_FULL) ? j : (int64_t)cand_idx[cand_off[b] + j];
      if (rr >= 0 && rr < nv) r = rr;
    }
    row_s[t] = r;
  }
  for (int x = t; x < HP * kIndexDim; x += kThreads) {
    const int h = x / kIndexDim, i = x % kIndexDim;
    q_s[h][i] = (h < hi) ? idx_q[((int64_t)b * hi + h) * kIndexDim + i] : 0.0f;
  }
  if (t < HP) w_s[t] = (t < hi) ? (idx_w ? idx_w[(int64_t)b * hi + t] : 1.0f) : 0.0f;
  __syncthreads();

  const float* kbase = idx_k + pool_row0[b] * kIndexDim;
  float4 v[kPieces];
#pragma unroll
  for (int it = 0; it < kPieces; ++it) {
    const int p = it * kThreads + t, r = p / kUnits, u = p % kUnits;
    const int64_t rr = row_s[r];
    v[it] = (rr >= 0) ? load_stream(kbase + rr * kIndexDim + u * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int it = 0; it < kPieces; ++it) {
    const int p = it * kThreads + t, r = p / kUnits, u = p % kUnits;
    *reinterpret_cast<float4*>(&k_s[r * kIndexDim + key_unit_swz(r, u) * 4]) = v[it];
  }
  __syncthreads();
  if (t >= kRows) return;
  const int64_t j = j0 + t;
  if (j >= n) return;
  float sc = -__builtin_inff();
  if (row_s[t] >= 0) {
    float acc[HP];
#pragma unroll
    for (int h = 0; h < HP; ++h) acc[h] = 0.0f;
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const float4 k4 = *reinterpret_cast<const float4*>(&k_s[t * kIndexDim + key_unit_swz(t, u) * 4]);
      const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = u * 4 + e;
#pragma unroll
        for (int h = 0; h < HP; ++h) acc[h] = __builtin_fmaf(q_s[h][i], kv[e], acc[h]);
      }
    }
    sc = finish_score(acc, w_s, HP, relu);
  }
  scores[(int64_t)b * stride + j] = sc;
}

// ---- decode, MXFP4 keys ------------------------------------------------------
constexpr int kMxRows = 64;                   // candidates per workgroup (one wave), one per thread
constexpr int kMxThreads = kMxRows;
constexpr int kMxRowB = kIndexDim / 2;        // 64 code bytes per key row
constexpr int kMxScales = kIndexDim / 32;     // 4 E8M0 scales per key row
static_assert(kMxScales == 4, "a key row's scales are read as one 32-bit word");

// 16-byte unit u of code row r sits at unit u ^ ((r >> 2) & 3): sixteen lanes
// reading the same unit of their own rows then cover all 64 banks.
__device__ __forceinline__ int mx_unit_swz(int r, int u) { return u ^ ((r >> 2) & 3); }

// ONE: a single index head (the workloads' form): q takes 512 B of LDS and each
// row is widened eight values at a time into its FMA chain, which keeps the
// footprint small enough for many workgroups per CU (more loads in flight).
template <bool ONE>
__global__ __launch_bounds__(kMxThreads) void index_scores_decode_mx(
    int32_t hi, int32_t relu, int32_t max_cand, const int64_t* __restrict__ pos,
    const int32_t* __restrict__ mode, const int32_t* __restrict__ ratio,
    const int64_t* __restrict__ pool_row0, const int32_t* __restrict__ pool_len,
    const int64_t* __restrict__ cand_off, const int32_t* __restrict__ cand_idx,
    const float* __restrict__ idx_q, const float* __restrict__ idx_w, const uint8_t* __restrict__ kcodes,
    const uint8_t* __restrict__ kscales, float* __restrict__ scores, int64_t stride) {
  __shared__ __attribute__((aligned(16))) uint8_t c_s[kMxRows * kMxRowB];
  __shared__ __attribute__((aligned(16))) float q_s[ONE ? 1 : kMaxIndexHeads][kIndexDim];
  __shared__ float w_s[ONE ? 1 : kMaxIndexHeads];
  const int b = blockIdx.y;
  const int t = threadIdx.x;
  const int md = mode[b];
  if (md != CSA2_MODE_FULL && md != CSA2_MODE_REINDEX) return;
  if (ONE) hi = 1;
  const int64_t nv = n_valid_of(pos[b], ratio[b], md, pool_len[b]);
  int64_t n = (md == CSA2_MODE_FULL) ? nv : (cand_off ? cand_off[b + 1] - cand_off[b] : 0);
  if (n > max_cand) n = max_cand;
  const int64_t j0 = (int64_t)blockIdx.x * kMxRows;
  if (j0 >= n) return;

  // candidate c of this workgroup -> its pool row, -1 when there is none
  const int64_t coff = (md == CSA2_MODE_REINDEX) ? cand_off[b] : 0;
  auto row_of = [&](int c) -> int64_t {
    const int64_t jj = j0 + c;
    if (jj >= n) return -1;
    const int64_t rr = (md == CSA2_MODE_FULL) ? jj : (int64_t)cand_idx[coff + jj];
    return (rr >= 0 && rr < nv) ? rr : -1;
  };
  const int64_t j = j0 + t;
  const int64_t my_row = row_of(t);
  const int64_t prow0 = pool_row0[b];
  // every global load of the workgroup is issued before its one barrier: the
  // code rows (four threads per 64-byte row, a quarter of the rows per pass),
  // this thread's four scale bytes, and q
  uint4 v[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = it * (kMxRows / 4) + (t >> 2), u = t & 3;
    const int64_t rr = row_of(r);
    v[it] = (rr >= 0) ? load_stream(kcodes + (prow0 + rr) * kMxRowB + u * 16) : make_uint4(0u, 0u, 0u, 0u);
  }
  const uint32_t sc4 = (my_row >= 0) ? *reinterpret_cast<const uint32_t*>(kscales + (prow0 + my_row) * kMxScales)
                                     : 0u;
  for (int x = t; x < hi * kIndexDim; x += kMxThreads)
    q_s[x / kIndexDim][x % kIndexDim] = idx_q[(int64_t)b * hi * kIndexDim + x];
  if (t < hi) w_s[t] = idx_w ? idx_w[(int64_t)b * hi + t] : 1.0f;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = it * (kMxRows / 4) + (t >> 2), u = t & 3;
    *reinterpret_cast<uint4*>(&c_s[r * kMxRowB + mx_unit_swz(r, u) * 16]) = v[it];
  }
  __syncthreads();
  if (j >= n) return;
  float sc = -__builtin_inff();
  if (ONE && my_row >= 0) {
    float acc = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // unit u = dims 32u .. 32u+31 = scale block u
      const uint4 c = *reinterpret_cast<const uint4*>(&c_s[t * kMxRowB + mx_unit_swz(t, u) * 16]);
      const uint32_t e = (sc4 >> (8 * u)) & 0xffu;
      const float scale = e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
      const uint32_t wds[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        float kv[8];
        fp4x8_to_f32x8(wds[wd], kv);
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) acc = __builtin_fmaf(q_s[0][32 * u + 8 * wd + e2], kv[e2] * scale, acc);
      }
    }
    if (relu) acc = acc > 0.0f ? acc : 0.0f;
    const float s = __builtin_fmaf(w_s[0], acc, 0.0f);
    sc = (s == 0.0f) ? 0.0f : s;
  } else if (!ONE && my_row >= 0) {
    // widen the row: unit u holds dims 32u .. 32u+31, the block of scale byte u
    float k[kIndexDim];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint4 c = *reinterpret_cast<const uint4*>(&c_s[t * kMxRowB + mx_unit_swz(t, u) * 16]);
      const uint32_t e = (sc4 >> (8 * u)) & 0xffu;
      // 2^(e-127) as fp32 (e = 0 is the subnormal 2^-127); products are exact
      const float scale = e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
      const uint32_t wds[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        float kv[8];
        fp4x8_to_f32x8(wds[wd], kv);
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) k[32 * u + 8 * wd + e2] = kv[e2] * scale;
      }
    }
    // heads in order, each folded into the score as soon as its chain ends
    float s = 0.0f;
#pragma unroll 1
    for (int h = 0; h < hi; ++h) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < kIndexDim; ++i) acc = __builtin_fmaf(q_s[h][i], k[i], acc);
      if (relu) acc = acc > 0.0f ? acc : 0.0f;
      s = __builtin_fmaf(w_s[h], acc, s);
    }
    sc = (s == 0.0f) ? 0.0f : s;
  }
  scores[(int64_t)b * stride + j] = sc;
}

// ---- prefill: queries x candidates, register tiled -------------------------
constexpr int kPQ = 128;  // queries per workgroup
constexpr int kPC = 128;  // candidates per workgroup
constexpr int kPK = 16;   // k slab

__global__ __launch_bounds__(256, 4) void index_scores_prefill(
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

  // loaders: 128 rows x 16 floats per slab = 512 float4, two per thread; the
  // next slab's loads are issued before the current slab's products
  float4 vq[2], vk[2];
  auto load = [&](int s) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int p = it * 256 + t;
      const int r = p >> 2, part = p & 3;
      const int qq = q0 + r, cc = c0 + r;
      vq[it] = (qq < T) ? *reinterpret_cast<const float4*>(idx_q + (int64_t)qq * kIndexDim + s * kPK + part * 4)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
      vk[it] = (cc < nmax) ? *reinterpret_cast<const float4*>(idx_k + (int64_t)cc * kIndexDim + s * kPK + part * 4)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto stage = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int p = it * 256 + t;
      const int r = p >> 2, part = p & 3;
      qs[part * 4 + 0][r] = vq[it].x;
      qs[part * 4 + 1][r] = vq[it].y;
      qs[part * 4 + 2][r] = vq[it].z;
      qs[part * 4 + 3][r] = vq[it].w;
      ks[part * 4 + 0][r] = vk[it].x;
      ks[part * 4 + 1][r] = vk[it].y;
      ks[part * 4 + 2][r] = vk[it].z;
      ks[part * 4 + 3][r] = vk[it].w;
    }
  };
  load(0);
  for (int s = 0; s < kIndexDim / kPK; ++s) {
    stage();
    __syncthreads();
    if (s + 1 < kIndexDim / kPK) load(s + 1);
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
                               const float* idx_w, const void* idx_k_v, const uint8_t* idx_k_scale,
                               float* scores, int64_t stride, hipStream_t s) {
  if (B == 0 || bt.max_candidates == 0) return hipSuccess;
  const int hi = d.index_heads;
  if (d.index_key_dtype == CSA2_IDXK_MXFP4) {
    dim3 grid((bt.max_candidates + kMxRows - 1) / kMxRows, B);
    const uint8_t* kc = static_cast<const uint8_t*>(idx_k_v);
    if (hi == 1)
      hipLaunchKernelGGL(index_scores_decode_mx<true>, grid, dim3(kMxThreads), 0, s, hi, d.index_relu,
                         bt.max_candidates, bt.pos, bt.mode, bt.compress_ratio, bt.pool_row0, bt.pool_len,
                         bt.cand_off, bt.cand_idx, idx_q, idx_w, kc, idx_k_scale, scores, stride);
    else
      hipLaunchKernelGGL(index_scores_decode_mx<false>, grid, dim3(kMxThreads), 0, s, hi, d.index_relu,
                         bt.max_candidates, bt.pos, bt.mode, bt.compress_ratio, bt.pool_row0, bt.pool_len,
                         bt.cand_off, bt.cand_idx, idx_q, idx_w, kc, idx_k_scale, scores, stride);
    return hipGetLastError();
  }
  const float* idx_k = static_cast<const float*>(idx_k_v);
  dim3 grid((bt.max_candidates + kRows - 1) / kRows, B);
#define CSA2_IDX_ARGS                                                                                 \
  hi, d.index_relu, bt.max_candidates, bt.pos, bt.mode, bt.compress_ratio, bt.pool_row0, bt.pool_len, \
      bt.cand_off, bt.cand_idx, idx_q, idx_w, idx_k, scores, stride
  if (hi <= 1)
    hipLaunchKernelGGL(index_scores_decode<1>, grid, dim3(kThreads), 0, s, CSA2_IDX_ARGS);
  else if (hi <= 4)
    hipLaunchKernelGGL(index_scores_decode<4>, grid, dim3(kThreads), 0, s, CSA2_IDX_ARGS);
  else if (hi <= 16)
    hipLaunchKernelGGL(index_scores_decode<16>, grid, dim3(kThreads), 0, s, CSA2_IDX_ARGS);
  else
    hipLaunchKernelGGL(index_scores_decode<64>, grid, dim3(kThreads), 0, s, CSA2_IDX_ARGS);
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
