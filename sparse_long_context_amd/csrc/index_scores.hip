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
//    reused across queries: 128 queries x 256 candidates per workgroup on the
//    matrix cores, whose single-rounding fp32 rank-1 updates run each output's
//    FMA chain over i in order.
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

struct DecodeIdxArgs {
  int32_t hi, relu, max_cand, B;
  const int64_t* pos;
  const int32_t* mode;
  const int32_t* ratio;
  const int64_t* pool_row0;
  const int32_t* pool_len;
  const int64_t* cand_off;
  const int32_t* cand_idx;
  const float* idx_q;
  const float* idx_w;
  const float* idx_k;
  float* scores;
  int64_t stride;
};

// Candidates a query scores (0 for Reuse / Window queries), and its reachable
// count.
__device__ __forceinline__ int64_t decode_cands(const DecodeIdxArgs& a, int b, int& md, int64_t& nv) {
  md = a.mode[b];
  nv = 0;
  if (md != CSA2_MODE_FULL && md != CSA2_MODE_REINDEX) return 0;
  nv = n_valid_of(a.pos[b], a.ratio[b], md, a.pool_len[b]);
  // a REINDEX query without lists (cand_off NULL) has an empty list
  int64_t n = (md == CSA2_MODE_FULL) ? nv : (a.cand_off ? a.cand_off[b + 1] - a.cand_off[b] : 0);
  return n > a.max_cand ? a.max_cand : n;
}

template <int HP>
struct DecodeTileLds {
  float k_s[kRows * kIndexDim];
  float q_s[HP][kIndexDim];
  float w_s[HP];
  int64_t row_s[kRows];
};

// Candidates j0 .. j0 + 31 of query b (the whole workgroup; two barriers): rows
// and the query into LDS, the 16 KiB of key rows through registers into the
// swizzled tile, then 32 lanes run one candidate's FMA chain each.
template <int HP>
__device__ __forceinline__ void decode_tile(const DecodeIdxArgs& a, DecodeTileLds<HP>& L, int b, int md,
                                            int64_t nv, int64_t n, int64_t j0) {
  const int t = threadIdx.x;
  if (t < kRows) {  // candidate rows (pool-relative), -1 when there is none
    const int64_t j = j0 + t;
    int64_t r = -1;
    if (j < n) {
      const int64_t rr = (md == CSA2_MODE_FULL) ? j : (int64_t)a.cand_idx[a.cand_off[b] + j];
      if (rr >= 0 && rr < nv) r = rr;
    }
    L.row_s[t] = r;
  }
  for (int x = t; x < HP * kIndexDim; x += kThreads) {
    const int h = x / kIndexDim, i = x % kIndexDim;
    L.q_s[h][i] = (h < a.hi) ? a.idx_q[((int64_t)b * a.hi + h) * kIndexDim + i] : 0.0f;
  }
  if (t < HP) L.w_s[t] = (t < a.hi) ? (a.idx_w ? a.idx_w[(int64_t)b * a.hi + t] : 1.0f) : 0.0f;
  __syncthreads();

  const float* kbase = a.idx_k + a.pool_row0[b] * kIndexDim;
  float4 v[kPieces];
#pragma unroll
  for (int it = 0; it < kPieces; ++it) {
    const int p = it * kThreads + t, r = p / kUnits, u = p % kUnits;
    const int64_t rr = L.row_s[r];
    v[it] = (rr >= 0) ? load_stream(kbase + rr * kIndexDim + u * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int it = 0; it < kPieces; ++it) {
    const int p = it * kThreads + t, r = p / kUnits, u = p % kUnits;
    *reinterpret_cast<float4*>(&L.k_s[r * kIndexDim + key_unit_swz(r, u) * 4]) = v[it];
  }
  __syncthreads();
  const int64_t j = j0 + t;
  if (t >= kRows || j >= n) return;
  float sc = -__builtin_inff();
  if (L.row_s[t] >= 0) {
    float acc[HP];
#pragma unroll
    for (int h = 0; h < HP; ++h) acc[h] = 0.0f;
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const float4 k4 = *reinterpret_cast<const float4*>(&L.k_s[t * kIndexDim + key_unit_swz(t, u) * 4]);
      const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = u * 4 + e;
#pragma unroll
        for (int h = 0; h < HP; ++h) acc[h] = __builtin_fmaf(L.q_s[h][i], kv[e], acc[h]);
      }
    }
    sc = finish_score(acc, L.w_s, HP, a.relu);
  }
  a.scores[(int64_t)b * a.stride + j] = sc;
}

// With one or a few index heads: eight waves per SIMD (at most 64 VGPRs), so
// eight workgroups per CU keep 128 KiB of key rows in flight, where the
// register use the compiler picks by itself (80) allows six.
//
// Grid (X, B): workgroup (x, b) scores tiles x, x + X, x + 2X, .. of query b.
// X covers every tile of lists up to kGridTiles tiles, so dense batches run
// one tile per workgroup; past that, a long list's workgroups loop, which
// keeps the grid (and the idle workgroups of the queries with short lists or
// none) from growing with the longest list of a ragged batch.
constexpr int kGridTiles = 512;  // 16,384 candidates
template <int HP, bool LOOP>  // LOOP: the grid is narrower than the longest list
__global__ __launch_bounds__(kThreads, (HP == 1 || (HP <= 4 && !LOOP)) ? 8 : 1) void index_scores_decode(
    DecodeIdxArgs a) {
  __shared__ __attribute__((aligned(16))) DecodeTileLds<HP> L;
  const int b = blockIdx.y;
  int md;
  int64_t nv;
  const int64_t n = decode_cands(a, b, md, nv);
  if constexpr (!LOOP) {
    const int64_t j0 = (int64_t)blockIdx.x * kRows;
    if (j0 >= n) return;  // whole workgroup, before any barrier
    decode_tile<HP>(a, L, b, md, nv, n, j0);
  } else {
    const int64_t step = (int64_t)gridDim.x * kRows;
#pragma clang loop unroll(disable)
    for (int64_t j0 = (int64_t)blockIdx.x * kRows; j0 < n; j0 += step) {  // uniform
      decode_tile<HP>(a, L, b, md, nv, n, j0);
      if (j0 + step < n) __syncthreads();  // this tile's LDS is read before the next one is written
    }
  }
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
      if (e - 2u <= 250u) {
        // 2 <= e <= 252: every key value code * 2^(e-127) is a finite normal
        // float, so the conversion applies the scale exactly, one instruction
        // per two values instead of a conversion and a multiply per value
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          float kv[8];
          fp4x8_pow2_to_f32x8(wds[wd], scale, kv);
#pragma unroll
          for (int e2 = 0; e2 < 8; ++e2) acc = __builtin_fmaf(q_s[0][32 * u + 8 * wd + e2], kv[e2], acc);
        }
      } else {
        // scale bytes 0, 1, 253, 254: products may be subnormal or overflow;
        // the exact code times the scale, rounded by the multiply
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          float kv[8];
          fp4x8_to_f32x8(wds[wd], kv);
#pragma unroll
          for (int e2 = 0; e2 < 8; ++e2) acc = __builtin_fmaf(q_s[0][32 * u + 8 * wd + e2], kv[e2] * scale, acc);
        }
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

// ---- decode, 17 .. 32 index heads (the pages' 32-head indexer) ------------
// One query's heads against 64 candidates per wave on the matrix cores: in
// v_mfma_f32_32x32x1_2b_f32, A is head h's query value at dim i (h = lane % 32,
// the same in both blocks) and B a candidate's key value at dim i (64
// candidates, 32 per block), so each element runs the fixed-order fmaf chain
// of its (head, candidate).  Heads past H_I are zero with zero weight.  A
// workgroup of four waves takes 256 candidates; key rows come in with
// coalesced 16-byte loads through LDS in slabs of 32 dims (whole 128-byte
// lines of each row), two slabs in flight, each with its 32 dims of the 32
// heads' queries (so LDS holds one slab of each, 42 KiB, and three
// workgroups share a CU).  The per-candidate sum over heads,
// in head order, needs the 32 heads of a candidate in one lane: lanes l and
// l + 32 hold complementary halves of the heads of candidates l % 32 (block 0)
// and 32 + l % 32 (block 1), and one permlane32 swap per register pair leaves
// lane l < 32 with all of block 0's and lane l + 32 with all of block 1's.
typedef float f32x32 __attribute__((ext_vector_type(32)));
constexpr int kHC = 256;           // candidates per workgroup
constexpr int kHS = 32;            // dims per slab
constexpr int kHU = kHS / 4;       // 16-byte units of a row per slab
constexpr int kHRow = kHS + 4;     // LDS row stride in floats (9 units: sixteen consecutive rows, one unit,
                                   // cover sixteen bank groups)
constexpr int kHKv = kHC * kHS / 4 / 256;  // float4 of keys per thread per slab (8)

__global__ __launch_bounds__(256, 3) void index_scores_decode_h32(
    int32_t hi, int32_t relu, int32_t max_cand, const int64_t* __restrict__ pos,
    const int32_t* __restrict__ mode, const int32_t* __restrict__ ratio,
    const int64_t* __restrict__ pool_row0, const int32_t* __restrict__ pool_len,
    const int64_t* __restrict__ cand_off, const int32_t* __restrict__ cand_idx,
    const float* __restrict__ idx_q, const float* __restrict__ idx_w, const float* __restrict__ idx_k,
    float* __restrict__ scores, int64_t stride) {
  __shared__ __attribute__((aligned(16))) float ks[kHC * kHRow];
  __shared__ __attribute__((aligned(16))) float qs[32 * kHRow];  // this slab's [head][i], zero past H_I
  __shared__ float w_s[32];
  __shared__ int32_t row_s[kHC];
  const int b = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int md = mode[b];
  if (md != CSA2_MODE_FULL && md != CSA2_MODE_REINDEX) return;
  const int64_t nv = n_valid_of(pos[b], ratio[b], md, pool_len[b]);
  int64_t n = (md == CSA2_MODE_FULL) ? nv : (cand_off ? cand_off[b + 1] - cand_off[b] : 0);
  if (n > max_cand) n = max_cand;
  const int64_t j0 = (int64_t)blockIdx.x * kHC;
  if (j0 >= n) return;

  {  // candidate rows (pool-relative), -1 when there is none
    const int64_t j = j0 + t;
    int32_t r = -1;
    if (j < n) {
      const int64_t rr = (md == CSA2_MODE_FULL) ? j : (int64_t)cand_idx[cand_off[b] + j];
      if (rr >= 0 && rr < nv) r = (int32_t)rr;  // pool rows fit 32 bits (pool_len is int32)
    }
    row_s[t] = r;
  }
  if (t < 32) w_s[t] = t < hi ? (idx_w ? idx_w[(int64_t)b * hi + t] : 1.0f) : 0.0f;
  __syncthreads();

  const float* kbase = idx_k + pool_row0[b] * kIndexDim;
  // two slabs in flight: slab s lands in vk[s % 2], its 32 dims of q (head
  // t / 8, dims 4 (t % 8) ..) in vq[s % 2]; the q slab is staged beside the
  // key slab, so LDS holds one slab of each (three workgroups per CU)
  float4 vk[2][kHKv], vq[2];
  auto load = [&](int sl, float4* v, float4& q) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < kHKv; ++it) {
      const int p = it * 256 + t, r = p / kHU, u = p % kHU;
      const int64_t rr = row_s[r];
      v[it] = rr >= 0 ? load_stream(kbase + rr * kIndexDim + sl * kHS + u * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const int h = t / kHU, u = t % kHU;
    q = h < hi ? *reinterpret_cast<const float4*>(idx_q + ((int64_t)b * hi + h) * kIndexDim + sl * kHS + 4 * u)
               : make_float4(0.f, 0.f, 0.f, 0.f);
  };
  auto stage = [&](const float4* v, const float4& q) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < kHKv; ++it) {
      const int p = it * 256 + t;
      *reinterpret_cast<float4*>(&ks[(p / kHU) * kHRow + 4 * (p % kHU)]) = v[it];
    }
    *reinterpret_cast<float4*>(&qs[(t / kHU) * kHRow + 4 * (t % kHU)]) = q;
  };
  f32x32 acc = f32x32{};
  const float* qa = &qs[(lane & 31) * kHRow];
  const float* kb = &ks[(64 * wv + lane) * kHRow];
  load(0, vk[0], vq[0]);
  load(1, vk[1], vq[1]);
#pragma unroll
  for (int sl = 0; sl < kIndexDim / kHS; ++sl) {
    stage(vk[sl & 1], vq[sl & 1]);
    __syncthreads();
    if (sl + 2 < kIndexDim / kHS) load(sl + 2, vk[sl & 1], vq[sl & 1]);
#pragma unroll
    for (int u = 0; u < kHU; ++u) {
      const float4 a4 = *reinterpret_cast<const float4*>(qa + 4 * u);
      const float4 b4 = *reinterpret_cast<const float4*>(kb + 4 * u);
      acc = __builtin_amdgcn_mfma_f32_32x32x1f32(a4.x, b4.x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x1f32(a4.y, b4.y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x1f32(a4.z, b4.z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x1f32(a4.w, b4.w, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  // D register r: block r / 16 (candidate 32 (r / 16) + lane % 32 of the
  // wave), head 8 ((r % 16) / 4) + 4 (lane / 32) + r % 4.  After the swaps,
  // mine[q] (q < 16) is head 8 (q / 4) + 4 upper + q % 4 and got[q] head
  // 8 (q / 4) + 4 (1 - upper) + q % 4 of this lane's candidate.
  const bool upper = lane >= 32;
  float mine[16], got[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[q]), __float_as_uint(acc[16 + q]), false,
                                                     false);
    // lanes < 32: sw[0] = own block-0 value, sw[1] = block-0 value of lane + 32;
    // lanes >= 32: sw[0] = block-1 value of lane - 32, sw[1] = own block-1 value
    mine[q] = __uint_as_float(upper ? sw[1] : sw[0]);
    got[q] = __uint_as_float(upper ? sw[0] : sw[1]);
  }
  float sc = 0.0f;
#pragma unroll
  for (int h = 0; h < 32; ++h) {
    const int q = 4 * (h / 8) + (h % 4);
    const bool second = ((h / 4) & 1) != 0;  // head in the +4 half
    float f = (second != upper) ? got[q] : mine[q];
    if (relu) f = f > 0.0f ? f : 0.0f;
    sc = __builtin_fmaf(w_s[h], f, sc);
  }
  sc = sc == 0.0f ? 0.0f : sc;
  const int c = 64 * wv + 32 * (upper ? 1 : 0) + (lane & 31);
  const int64_t j = j0 + c;
  if (j < n) scores[(int64_t)b * stride + j] = row_s[c] >= 0 ? sc : -__builtin_inff();
}

// ---- prefill: queries x candidates on the matrix cores ---------------------
// v_mfma_f32_32x32x1_2b_f32 is a rank-1 update D += a b^T of two 32 x 32 fp32
// blocks, each element one fused multiply-add with a single rounding: a chain
// of them over i = 0 .. 127 performs, per output, exactly the fmaf chain that
// defines the score (checked bit for bit on the GPU against the VALU chain,
// denormal and cancelling inputs included), at 32 fused operations per clock
// per SIMD against the VALU's 16.
//
// Tiles of 128 queries x 256 candidates; each of the four waves takes 64
// queries (the two blocks: A is a query's value at dim i) x 128 candidates
// (four accumulator sets: in set g, column n is candidate 4 n + g, so a lane
// ends up holding four consecutive scores of a row and stores them with one
// 16-byte store).  The operands stream through LDS in slabs of 16 dims.  Two
// resident workgroups per CU walk the tiles, so one's waits hide behind the
// other's products; every slab's global loads (the next tile's first slab
// included) are issued before the current slab's products, the barriers order
// LDS only, and a tile's scores are stored during the next tile's first slab.
// (A wave that has stores in flight waits for all of them with any later
// load: gfx9 counts loads and stores together and they may complete out of
// order, so only the other workgroup's products cover that drain.)
constexpr int kPQ = 128;            // queries per tile
constexpr int kPC = 256;            // candidates per tile
constexpr int kPS = 16;             // dims per slab
constexpr int kPSlabs = kIndexDim / kPS;
constexpr int kPU = kPS / 4;        // 16-byte units of a row per slab
constexpr int kPRow = kPS + 4;      // LDS row stride in floats (an odd number of units)
constexpr int kPQv = kPQ * kPS / 4 / 256;  // float4 of q per thread per slab (4)
constexpr int kPKv = kPC * kPS / 4 / 256;  // float4 of keys per thread per slab (8)

// Key rows keep their 16-byte unit u at u ^ ((r >> 4) & 3): with an odd row
// stride in units, the sixteen lanes of a read phase (rows 4 l + g, l < 16,
// one unit) then hit sixteen distinct bank groups; query rows are read sixteen
// consecutive rows at a time, which the odd stride alone spreads.
__device__ __forceinline__ int key_unit(int r, int u) { return u ^ ((r >> 4) & 3); }

// LDS writes of every wave visible to every wave, without waiting for this
// wave's outstanding global loads and stores
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// RELU: f = max(., 0); WEIGHTED: per-query weights (else w = 1, and
// fmaf(1, f, +0) = f + 0, which only turns -0 into +0)
template <bool RELU, bool WEIGHTED>
__global__ __launch_bounds__(256, 2) void index_scores_prefill(
    int32_t T, const int64_t* __restrict__ pos, int32_t md, int32_t ratio, int32_t pool_len,
    const float* __restrict__ idx_q, const float* __restrict__ idx_w,
    const float* __restrict__ idx_k, float* __restrict__ scores, int64_t stride, int32_t n_ct, int32_t n_tiles) {
  __shared__ __attribute__((aligned(16))) float qs[kPQ * kPRow];
  __shared__ __attribute__((aligned(16))) float ks[kPC * kPRow];
  __shared__ int32_t nv_s[2][kPQ];  // per tile parity: reachable count of each query
  __shared__ float w_s[2][kPQ];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int wq = (wv >> 1) * 64, wc = (wv & 1) * 128;

  // tile k of this workgroup: query tile (id / n_ct), candidate tile (id % n_ct);
  // a tile whose first candidate no query of it reaches is skipped whole
  auto tile_of = [&](int k) -> int { return (int)blockIdx.x + k * (int)gridDim.x; };
  auto tile_live = [&](int id, int& q0, int& c0, int64_t& nmax) -> bool {
    q0 = (id / n_ct) * kPQ;
    c0 = (id % n_ct) * kPC;
    const int qlast = (q0 + kPQ < T ? q0 + kPQ : T) - 1;
    nmax = n_valid_of(pos[qlast], ratio, md, pool_len);  // the tile's last query reaches furthest
    return c0 < nmax;
  };
  auto next_live = [&](int k, int& q0, int& c0, int64_t& nmax) -> int {
    for (; tile_of(k) < n_tiles; ++k)
      if (tile_live(tile_of(k), q0, c0, nmax)) return k;
    return -1;
  };

  float4 vq[kPQv], vk[kPKv];
  auto load = [&](int q0, int c0, int64_t nmax, int sl) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < kPQv; ++it) {
      const int p = it * 256 + t, r = p / kPU, part = p % kPU, qq = q0 + r;
      vq[it] = (qq < T) ? *reinterpret_cast<const float4*>(idx_q + (int64_t)qq * kIndexDim + sl * kPS + part * 4)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int it = 0; it < kPKv; ++it) {
      const int p = it * 256 + t, r = p / kPU, part = p % kPU, cc = c0 + r;
      vk[it] = (cc < nmax) ? *reinterpret_cast<const float4*>(idx_k + (int64_t)cc * kIndexDim + sl * kPS + part * 4)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto stage = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < kPQv; ++it) {
      const int p = it * 256 + t;
      *reinterpret_cast<float4*>(&qs[(p / kPU) * kPRow + (p % kPU) * 4]) = vq[it];
    }
#pragma unroll
    for (int it = 0; it < kPKv; ++it) {
      const int p = it * 256 + t, r = p / kPU;
      *reinterpret_cast<float4*>(&ks[r * kPRow + key_unit(r, p % kPU) * 4]) = vk[it];
    }
  };

  // this lane's operand rows: query wq + lane; candidates wc + 4 (lane % 32) + g
  const float* qa = &qs[(wq + lane) * kPRow];
  const int kr = wc + 4 * (lane & 31);
  const float* kb = &ks[kr * kPRow];
  const int ksw = (kr >> 4) & 3;  // the same swizzle for the four rows kr .. kr + 3

  f32x32 acc[4];
  // Scores of a finished tile (accumulators of the tile at q0p / c0p, its
  // counts and weights in slot pp).  Positions ascend with the query in a
  // chunk, so the tile's first query reaches least: when it reaches all 256
  // candidates (nearly every tile) no score is tested.  D of set g, register
  // r: block r / 16 (queries wq + 32 (r / 16) ..), row 8 ((r % 16) / 4) +
  // 4 (lane / 32) + r % 4, column lane % 32 (candidate wc + 4 (lane % 32) + g).
  auto store_tile = [&](int q0p, int c0p, int pp) __attribute__((always_inline)) {
    // buffer stores from one descriptor per tile, at 32-bit byte offsets
    // within it (the lane's first row and its four candidates, plus the row);
    // the descriptor spans the tile's rows (the launcher keeps 128 rows x
    // stride x 4 B below 2^32)
    const int rows = T - q0p < kPQ ? T - q0p : kPQ;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        scores + (int64_t)q0p * stride + c0p, (short)0, rows > 0 ? (int32_t)((uint32_t)rows * (uint32_t)stride * 4u) : 0,
        0x00020000);
    const int lane_off = (int)(((uint32_t)(wq + 4 * (lane >> 5)) * (uint32_t)stride + (uint32_t)kr) * 4u);
    // the row stride in bytes, opaque here, so the 32 row offsets are formed
    // per store instead of being hoisted out of the tile loop into 32 live
    // registers
    uint32_t rstride = (uint32_t)stride * 4u;
    asm volatile("" : "+s"(rstride));
    auto score_of = [&](float a, int qt) __attribute__((always_inline)) -> float {
      if (RELU) a = fmaxf(a, 0.0f);
      if (!WEIGHTED) return a + 0.0f;
      const float sc = __builtin_fmaf(w_s[pp][qt], a, 0.0f);
      return sc == 0.0f ? 0.0f : sc;
    };
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    if (nv_s[pp][0] >= c0p + kPC && q0p + kPQ <= T) {
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        const int row = 32 * (r >> 4) + 8 * ((r & 15) >> 2) + (r & 3);
        const int qt = wq + row + 4 * (lane >> 5);
        const u32x4 v = {__float_as_uint(score_of(acc[0][r], qt)), __float_as_uint(score_of(acc[1][r], qt)),
                         __float_as_uint(score_of(acc[2][r], qt)), __float_as_uint(score_of(acc[3][r], qt))};
        // the row's offset goes into the VGPR offset, not the SGPR one: with a
        // register soffset the compiler inserts no wait state between this
        // 16-byte store and the next write of its data registers, and the
        // store then picked up the next row's first value (seen on gfx950)
        __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, lane_off + (int)((uint32_t)row * rstride), 0, 0);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        const int row = 32 * (r >> 4) + 8 * ((r & 15) >> 2) + (r & 3);
        const int qt = wq + row + 4 * (lane >> 5);
        const int nvq = nv_s[pp][qt] - (c0p + kr);  // candidates of this lane's four the query reaches
        const int roff = lane_off + (int)((uint32_t)row * rstride);
#pragma unroll
        for (int g = 0; g < 4; ++g)
          if (g < nvq)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(score_of(acc[g][r], qt)), rsrc, roff + 4 * g, 0, 0);
      }
      // up to 128 stores: more than the 6-bit store count of a later wait can
      // leave in flight, so the rare edge tile drains its own (vmcnt(0) only)
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
  };

  int q0, c0;
  int64_t nmax;
  int k = next_live(0, q0, c0, nmax);
  if (k < 0) return;
  load(q0, c0, nmax, 0);
  // the tile whose scores are still in the accumulators; before the first
  // tile a placeholder whose queries reach nothing (slot 1 counts all 0), so
  // its store writes nothing and every tile's store runs the same code
  int q0p = T, c0p = 0;
  if (t < kPQ) nv_s[1][t] = 0;
  for (int par = 0; k >= 0; par ^= 1) {
    if (t < kPQ) {
      const int qq = q0 + t;
      nv_s[par][t] = qq < T ? (int32_t)n_valid_of(pos[qq], ratio, md, pool_len) : 0;
      if (WEIGHTED) w_s[par][t] = qq < T ? idx_w[qq] : 1.0f;
    }
    int nq0 = 0, nc0 = 0;
    int64_t nnmax = 0;
    const int kn = next_live(k + 1, nq0, nc0, nnmax);
    for (int sl = 0; sl < kPSlabs; ++sl) {
      stage();
      lds_barrier();
      if (sl + 1 < kPSlabs)
        load(q0, c0, nmax, sl + 1);
      else if (kn >= 0)
        load(nq0, nc0, nnmax, 0);
      if (sl == 0) {
        // the previous tile's stores go out after this tile's second-slab
        // loads, so waiting for those loads never waits for the stores
        store_tile(q0p, c0p, par ^ 1);
#pragma unroll
        for (int g = 0; g < 4; ++g) acc[g] = f32x32{};
      }
#pragma unroll
      for (int u = 0; u < kPS / 4; ++u) {
        const float4 a4 = *reinterpret_cast<const float4*>(qa + 4 * u);
        float4 b4[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) b4[g] = *reinterpret_cast<const float4*>(kb + g * kPRow + 4 * (u ^ ksw));
        const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float bv = j == 0 ? b4[g].x : j == 1 ? b4[g].y : j == 2 ? b4[g].z : b4[g].w;
            acc[g] = __builtin_amdgcn_mfma_f32_32x32x1f32(av[j], bv, acc[g], 0, 0, 0);
          }
        }
      }
      lds_barrier();
    }
    q0p = q0;
    c0p = c0;
    k = kn;
    q0 = nq0;
    c0 = nc0;
    nmax = nnmax;
    if (k < 0) store_tile(q0p, c0p, par);
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
  if (hi > 16 && hi <= 32) {
    hipLaunchKernelGGL(index_scores_decode_h32, dim3((bt.max_candidates + kHC - 1) / kHC, B), dim3(256), 0, s, hi,
                       d.index_relu, bt.max_candidates, bt.pos, bt.mode, bt.compress_ratio, bt.pool_row0,
                       bt.pool_len, bt.cand_off, bt.cand_idx, idx_q, idx_w, idx_k, scores, stride);
    return hipGetLastError();
  }
  DecodeIdxArgs a{hi, d.index_relu, bt.max_candidates, B, bt.pos, bt.mode, bt.compress_ratio, bt.pool_row0,
                  bt.pool_len, bt.cand_off, bt.cand_idx, idx_q, idx_w, idx_k, scores, stride};
  const int32_t tiles = (bt.max_candidates + kRows - 1) / kRows;
  const bool loop = tiles > kGridTiles;
  const dim3 grid((unsigned)(loop ? kGridTiles : tiles), (unsigned)B);
#define CSA2_IDX_LAUNCH(H)                                                                  \
  do {                                                                                       \
    if (loop) hipLaunchKernelGGL((index_scores_decode<H, true>), grid, dim3(kThreads), 0, s, a); \
    else hipLaunchKernelGGL((index_scores_decode<H, false>), grid, dim3(kThreads), 0, s, a);     \
  } while (0)
  if (hi <= 1) CSA2_IDX_LAUNCH(1);
  else if (hi <= 4) CSA2_IDX_LAUNCH(4);
  else if (hi <= 16) CSA2_IDX_LAUNCH(16);
  else CSA2_IDX_LAUNCH(64);
#undef CSA2_IDX_LAUNCH
  return hipGetLastError();
}

hipError_t launch_index_scores_prefill(const csa2_dims& d, int32_t T, const int64_t* pos, int32_t mode,
                                       int32_t ratio, int32_t pool_len, const float* idx_q,
                                       const float* idx_w, const float* idx_k, float* scores,
                                       int64_t stride, hipStream_t s) {
  if (T == 0 || pool_len == 0) return hipSuccess;
  const int32_t n_ct = (pool_len + kPC - 1) / kPC;
  const int32_t n_tiles = n_ct * ((T + kPQ - 1) / kPQ);
  const int n_cu = device_cu_count();
  const int grid = n_tiles < 2 * n_cu ? n_tiles : 2 * n_cu;  // two resident workgroups per CU
#define CSA2_PF_LAUNCH(R, W)                                                                                \
  hipLaunchKernelGGL((index_scores_prefill<R, W>), dim3(grid), dim3(256), 0, s, T, pos, mode, ratio, pool_len, \
                     idx_q, idx_w, idx_k, scores, stride, n_ct, n_tiles)
  if (d.index_relu) {
    if (idx_w) CSA2_PF_LAUNCH(true, true);
    else CSA2_PF_LAUNCH(true, false);
  } else {
    if (idx_w) CSA2_PF_LAUNCH(false, true);
    else CSA2_PF_LAUNCH(false, false);
  }
#undef CSA2_PF_LAUNCH
  return hipGetLastError();
}

}  // namespace csa2
