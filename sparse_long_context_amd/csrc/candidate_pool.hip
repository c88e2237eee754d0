// Hierarchical candidate pool (Reading Notes of DeepSeek-V4.1-Flash, section
// 3f C3: the Full layer scores each block of consecutive positions by its best
// member and keeps the best blocks as the pool later Reindex layers search;
// PocketLLM "DeepSeek-V4.1-Flash", "The CSA2 attention layers": the block a
// query is still filling is pinned into the pool, since its best member can
// lose to an older full block although it holds the newest entries).
//
// Three launches per batch, all per query:
//  1. block scores: the maximum of each block's reachable scores; the
//     still-filling block (the last one when n is not a multiple of the block
//     size) scores +inf, above every finite score, which is what pins it;
//  2. the top-K selection kernel over the block scores with K = top_blocks:
//     (score desc, block asc), emitted ascending, -1 padded;
//  3. expansion: each chosen block becomes its reachable entries; since the
//     chosen blocks ascend and only the last block can be partial, the list is
//     the pool in ascending order followed by -1s.
#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr size_t kWsAlign = 256;
size_t ws_align(size_t x) { return (x + kWsAlign - 1) & ~(kWsAlign - 1); }

struct PoolWs {
  float* bscore;       // [B][bstride]
  int64_t* pos;        // [B] nblk - 1
  int32_t* mode;       // [B] FULL, or WINDOW to skip the query
  int32_t* ratio;      // [B] 1
  int32_t* pool_len;   // [B] nblk
  int32_t* sel;        // [B][top_blocks] chosen blocks
  int64_t bstride;
};

int64_t max_blocks(int32_t max_cand, int32_t bs) { return ((int64_t)max_cand + bs - 1) / bs; }

PoolWs carve(void* ws, int32_t B, int32_t max_cand, int32_t bs, int32_t top_blocks) {
  PoolWs w;
  uint8_t* p = static_cast<uint8_t*>(ws);
  w.bstride = (int64_t)(ws_align((size_t)max_blocks(max_cand, bs) * sizeof(float)) / sizeof(float));
  w.bscore = reinterpret_cast<float*>(p);
  p += ws_align((size_t)B * (size_t)w.bstride * sizeof(float));
  w.pos = reinterpret_cast<int64_t*>(p);
  p += ws_align((size_t)B * sizeof(int64_t));
  w.mode = reinterpret_cast<int32_t*>(p);
  p += ws_align((size_t)B * sizeof(int32_t));
  w.ratio = reinterpret_cast<int32_t*>(p);
  p += ws_align((size_t)B * sizeof(int32_t));
  w.pool_len = reinterpret_cast<int32_t*>(p);
  p += ws_align((size_t)B * sizeof(int32_t));
  w.sel = reinterpret_cast<int32_t*>(p);
  return w;
}

__device__ __forceinline__ int64_t pool_n(int b, const int64_t* pos, const int32_t* mode, const int32_t* ratio,
                                          const int32_t* pool_len, int32_t max_cand) {
  if (mode[b] != CSA2_MODE_FULL) return -1;
  int64_t n = n_valid_of(pos[b], ratio[b], CSA2_MODE_FULL, pool_len[b]);
  return n < max_cand ? n : (int64_t)max_cand;
}

__global__ __launch_bounds__(256) void pool_block_scores(int32_t max_cand, int32_t bs, const int64_t* __restrict__ pos,
                                                         const int32_t* __restrict__ mode,
                                                         const int32_t* __restrict__ ratio,
                                                         const int32_t* __restrict__ pool_len,
                                                         const float* __restrict__ scores, int64_t stride,
                                                         PoolWs w) {
  const int b = blockIdx.y;
  const int64_t n = pool_n(b, pos, mode, ratio, pool_len, max_cand);
  const int64_t nblk = n > 0 ? (n + bs - 1) / bs : 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    w.pos[b] = nblk - 1;
    w.mode[b] = nblk > 0 ? CSA2_MODE_FULL : CSA2_MODE_WINDOW;
    w.ratio[b] = 1;
    w.pool_len[b] = (int32_t)nblk;
  }
  const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (blk >= nblk) return;
  const float* sc = scores + (int64_t)b * stride;
  const int64_t lo = blk * bs;
  const int64_t hi = (lo + bs < n) ? lo + bs : n;
  float m = -__builtin_inff();
  for (int64_t i = lo; i < hi; ++i) m = fmaxf(m, sc[i]);
  if (hi - lo < bs) m = __builtin_inff();  // the block still being filled: pinned
  w.bscore[(int64_t)b * w.bstride + blk] = m;
}

__global__ __launch_bounds__(256) void pool_expand(int32_t B, int32_t max_cand, int32_t bs, int32_t top_blocks,
                                                   const int64_t* __restrict__ pos, const int32_t* __restrict__ mode,
                                                   const int32_t* __restrict__ ratio,
                                                   const int32_t* __restrict__ pool_len, PoolWs w,
                                                   int64_t* __restrict__ cand_off, int32_t* __restrict__ cand_idx) {
  const int b = blockIdx.y;
  const int64_t cap = (int64_t)top_blocks * bs;
  const int64_t n = pool_n(b, pos, mode, ratio, pool_len, max_cand);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    cand_off[b] = (int64_t)b * cap;
    if (b == B - 1) cand_off[B] = (int64_t)B * cap;
  }
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= cap) return;
  int32_t v = -1;
  if (n > 0) {
    const int32_t blk = w.sel[(int64_t)b * top_blocks + i / bs];
    if (blk >= 0) {
      const int64_t p = (int64_t)blk * bs + i % bs;
      if (p < n) v = (int32_t)p;
    }
  }
  cand_idx[(int64_t)b * cap + i] = v;
}

}  // namespace

size_t candidate_pool_ws_bytes(int32_t B, int32_t max_cand, int32_t bs, int32_t top_blocks) {
  const size_t bstride = ws_align((size_t)max_blocks(max_cand, bs) * sizeof(float)) / sizeof(float);
  return ws_align((size_t)B * bstride * sizeof(float)) + ws_align((size_t)B * sizeof(int64_t)) +
         3 * ws_align((size_t)B * sizeof(int32_t)) + ws_align((size_t)B * (size_t)top_blocks * sizeof(int32_t));
}

hipError_t launch_candidate_pool(int32_t B, const csa2_batch& bt, const float* scores, int64_t stride,
                                 int32_t bs, int32_t top_blocks, int64_t* cand_off, int32_t* cand_idx, void* ws,
                                 hipStream_t s) {
  if (B == 0) return hipSuccess;
  const int32_t max_cand = bt.max_candidates;
  PoolWs w = carve(ws, B, max_cand, bs, top_blocks);
  const int64_t nblk_max = max_blocks(max_cand, bs);
  if (nblk_max > 0) {
    hipLaunchKernelGGL(pool_block_scores, dim3((unsigned)((nblk_max + 255) / 256), B), dim3(256), 0, s, max_cand,
                       bs, bt.pos, bt.mode, bt.compress_ratio, bt.pool_len, scores, stride, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    csa2_batch blk{};
    blk.pos = w.pos;
    blk.mode = w.mode;
    blk.compress_ratio = w.ratio;
    blk.pool_len = w.pool_len;
    blk.max_candidates = (int32_t)nblk_max;
    e = launch_topk_k(top_blocks, B, blk, w.bscore, w.bstride, w.sel, s);
    if (e != hipSuccess) return e;
  }
  const int64_t cap = (int64_t)top_blocks * bs;
  hipLaunchKernelGGL(pool_expand, dim3((unsigned)((cap + 255) / 256), B), dim3(256), 0, s, B, max_cand, bs,
                     top_blocks, bt.pos, bt.mode, bt.compress_ratio, bt.pool_len, w, cand_off, cand_idx);
  return hipGetLastError();
}

}  // namespace csa2
