// Top-K selection (Reading Notes of DeepSeek-V4.1-Flash, section 3f C2 Step 2:
// keep the K best-scoring entries; PocketLLM "DeepSeek-V4.1-Flash",
// "Correctness and precision": unused slots hold -1).
//
// Order: score descending, then row ascending (the lowest row wins a tie); +0
// and -0 tie.  Output: the chosen rows in ascending order, then -1s.
//
// One workgroup (1024 threads, 16 waves) per query.  Scores map to
// order-preserving 32-bit keys; ineligible slots get key 0, below every finite
// score and -inf.  Up to 16,384 candidates the keys live in registers (thread t
// holds the contiguous run [t*kpt, t*kpt+kpt)), and the selection is:
//  1. one LDS histogram of the top 12 key bits and a block-wide suffix scan
//     find the bucket that holds the K-th best key and how many keys lie above
//     it (and the eligible total: at most K eligible means take them all);
//  2. the keys of that bucket (typically 1-2 % of them) are gathered into LDS
//     and ranked exactly against each other under (key desc, row asc); the
//     bucket keys ranked below the remaining quota are marked in an LDS bitmap;
//  3. compaction: a key is chosen if its bucket lies above the boundary bucket
//     or it is marked; one block-wide prefix over threads (= index order) of
//     the per-thread counts places every chosen row.
// When the boundary bucket is too large to rank (heavy ties), or the list is
// longer than 16,384, a three-digit radix select (bits 31-20, 19-8, 7-0) finds
// the exact K-th key instead, with the keys re-read from the score buffer for
// long lists.
#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxKpt = 16;              // keys per thread held in registers
static_assert(kMaxKpt == 16, "a thread's marks are read as one 16-bit run of a 32-bit word");
constexpr int kRegKeys = kThreads * kMaxKpt;
constexpr int kBins = 4096;

__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;  // -0 ties with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (1ull << lane) - 1ull; }

// Inclusive prefix sum over the 64 lanes of a wave: shifts within each row of
// 16 lanes, then the last lane of a row is broadcast into the rows above it
// (DPP row_shr:1,2,4,8, row_bcast:15, row_bcast:31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);
  return (uint32_t)x;
}

// Block-wide exclusive suffix sum (sum over threads with a larger id).  Every
// call site passes a barrier before red_s is written again.
__device__ __forceinline__ uint32_t block_suffix_excl(uint32_t v, uint32_t* red_s, int lane, int wv) {
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) red_s[wv] = inc;
  __syncthreads();
  uint32_t higher = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t c = red_s[w];
    higher += (w > wv) ? c : 0u;
    total += (w == wv) ? c : 0u;
  }
  // within the wave: lanes above this one hold (wave total - inclusive prefix)
  return higher + (total - inc);
}

// Block-wide exclusive prefix sums of two values (sum over threads with a
// smaller id); also returns the totals.  Every call site passes a barrier
// before red_s is written again.
__device__ __forceinline__ void block_prefix2(uint32_t a, uint32_t b, uint32_t* red_s, int lane, int wv,
                                              uint32_t& pa, uint32_t& pb, uint32_t& ta, uint32_t& tb) {
  const uint32_t ia = wave_incl_scan(a), ib = wave_incl_scan(b);
  if (lane == 63) red_s[wv] = ia, red_s[kWaves + wv] = ib;
  __syncthreads();
  uint32_t la = 0, lb = 0;
  ta = 0, tb = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t ca = red_s[w], cb = red_s[kWaves + w];
    if (w < wv) la += ca, lb += cb;
    ta += ca, tb += cb;
  }
  pa = la + ia - a;
  pb = lb + ib - b;
}

constexpr int kRankCap = 1024;  // boundary-bucket keys ranked directly
constexpr int kMaxBpt = kBins / kThreads;  // histogram buckets owned per thread (>= 1)

// Find the bucket of an nb-bucket histogram that holds the krem-th largest
// key: each thread owns a run of consecutive buckets, a block-wide suffix scan
// gives the count above each run.  pick_s[0] = bucket, pick_s[1] = keys above
// it, pick_s[2] = all keys counted.  Contains barriers; call uniformly.
__device__ __forceinline__ void find_bucket(const uint32_t* hist_s, int nb, uint32_t krem, uint32_t* red_s,
                                            uint32_t* pick_s, int t, int lane, int wv) {
  const int bpt = (nb + kThreads - 1) / kThreads;
  uint32_t c[kMaxBpt], tot = 0;
#pragma unroll
  for (int u = 0; u < kMaxBpt; ++u) {
    const int bkt = t * bpt + u;
    c[u] = (u < bpt && bkt < nb) ? hist_s[bkt] : 0u;
    tot += c[u];
  }
  uint32_t above = block_suffix_excl(tot, red_s, lane, wv);
  if (t == 0) pick_s[2] = above + tot;
#pragma unroll
  for (int u = kMaxBpt - 1; u >= 0; --u) {
    if (u < bpt) {
      if (above < krem && krem <= above + c[u]) {
        pick_s[0] = t * bpt + u;
        pick_s[1] = above;
      }
      above += c[u];
    }
  }
}

// Radix select over digits d0 .. 2 (bits 31-20, 19-8, 7-0) starting from a
// known prefix; `count_keys(shift, nb, prefix, pmask)` adds the keys matching
// the prefix into hist_s.  Returns the K-th key and the quota left among keys
// equal to it.
template <typename CountFn>
__device__ __forceinline__ void radix_finish(int d0, uint32_t prefix, uint32_t pmask, uint32_t krem,
                                             uint32_t* hist_s, uint32_t* red_s, uint32_t* pick_s, int t,
                                             int lane, int wv, CountFn count_keys, uint32_t& thr,
                                             uint32_t& take_eq) {
#pragma unroll 1
  for (int d = d0; d < 3; ++d) {
    const int shift = d == 0 ? 20 : (d == 1 ? 8 : 0);
    const int nb = d == 2 ? 256 : 4096;
    const uint32_t dm = (uint32_t)(nb - 1);
    for (int x = t; x < nb; x += kThreads) hist_s[x] = 0u;
    __syncthreads();
    count_keys(shift, dm, prefix, pmask);
    __syncthreads();
    find_bucket(hist_s, nb, krem, red_s, pick_s, t, lane, wv);
    __syncthreads();
    krem -= pick_s[1];
    prefix |= pick_s[0] << shift;
    pmask |= dm << shift;
    __syncthreads();
  }
  thr = prefix;
  take_eq = krem;
}

__global__ __launch_bounds__(kThreads) void topk_kernel(
    int32_t K, int32_t max_cand, const int64_t* __restrict__ pos, const int32_t* __restrict__ mode,
    const int32_t* __restrict__ ratio, const int32_t* __restrict__ pool_len,
    const int64_t* __restrict__ cand_off, const int32_t* __restrict__ cand_idx,
    const float* __restrict__ scores, int64_t stride, int32_t* __restrict__ topk_idx) {
  __shared__ __attribute__((aligned(16))) uint32_t hist_s[kBins];
  __shared__ uint32_t red_s[2 * kWaves];
  __shared__ uint32_t pick_s[4];
  __shared__ uint64_t bk_s[kRankCap];           // boundary-bucket (key << 32 | ~index)
  __shared__ uint32_t mark_s[kRegKeys / 32];    // chosen boundary-bucket keys, by index
  __shared__ uint32_t bcount_s;

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
  int32_t* out = topk_idx + (int64_t)b * K;

  auto row_of = [&](int i) -> int32_t { return lst ? lst[i] : i; };
  auto key_global = [&](int i) -> uint32_t {
    const int32_t r = row_of(i);
    return (r >= 0 && r < nv) ? order_key(sc[i]) : 0u;
  };
  auto pad = [&](uint32_t chosen) {
    if (chosen > (uint32_t)K) chosen = K;
    for (int x = (int)chosen + t; x < K; x += kThreads) out[x] = -1;
  };

  if (n > kRegKeys) {
    // ---- long lists: full radix select, keys re-read from the score buffer ----
    uint32_t my_elig = 0;
    for (int i = t; i < n; i += kThreads) my_elig += (key_global(i) != 0u);
    const uint32_t incl = block_suffix_excl(my_elig, red_s, lane, wv) + my_elig;
    if (t == 0) pick_s[2] = incl;
    __syncthreads();
    const uint32_t total = pick_s[2];
    __syncthreads();
    uint32_t thr = 0, take_eq = 0;
    if (total > (uint32_t)K)
      radix_finish(0, 0u, 0u, (uint32_t)K, hist_s, red_s, pick_s, t, lane, wv,
                   [&](int shift, uint32_t dm, uint32_t prefix, uint32_t pmask) {
                     for (int i = t; i < n; i += kThreads) {
                       const uint32_t kk = key_global(i);
                       if (kk != 0u && (kk & pmask) == prefix) atomicAdd(&hist_s[(kk >> shift) & dm], 1u);
                     }
                   },
                   thr, take_eq);
    const bool has_eq = thr != 0u;
    const int seg = ((n + kWaves - 1) / kWaves + 63) & ~63;
    const int s0 = wv * seg, s1 = (s0 + seg < n) ? s0 + seg : n;
    uint32_t cnt_gt = 0, cnt_eq = 0;
    for (int q0 = s0; q0 < s1; q0 += 64) {
      const int i = q0 + lane;
      const uint32_t kk = (i < s1) ? key_global(i) : 0u;
      cnt_gt += __popcll(__ballot(i < s1 && kk > thr));
      cnt_eq += __popcll(__ballot(i < s1 && has_eq && kk == thr));
    }
    uint32_t gt_run, eq_run, gt_tot, eq_tot;
    block_prefix2(lane == 0 ? cnt_gt : 0u, lane == 0 ? cnt_eq : 0u, red_s, lane, wv, gt_run, eq_run, gt_tot,
                  eq_tot);
    gt_run = __shfl(gt_run, 0);
    eq_run = __shfl(eq_run, 0);
    for (int q0 = s0; q0 < s1; q0 += 64) {
      const int i = q0 + lane;
      const uint32_t kk = (i < s1) ? key_global(i) : 0u;
      const bool gt = i < s1 && kk > thr;
      const bool eq = i < s1 && has_eq && kk == thr;
      const uint64_t bg = __ballot(gt), be = __ballot(eq);
      const uint32_t gtb = gt_run + __popcll(bg & lanemask_lt(lane));
      const uint32_t eqb = eq_run + __popcll(be & lanemask_lt(lane));
      if (gt || (eq && eqb < take_eq)) {
        const uint32_t p = gtb + (eqb < take_eq ? eqb : take_eq);
        if (p < (uint32_t)K) out[p] = row_of(i);
      }
      gt_run += __popcll(bg);
      eq_run += __popcll(be);
    }
    pad(gt_tot + (eq_tot < take_eq ? eq_tot : take_eq));
    return;
  }

  // ---- keys in registers ----
  constexpr int kpt = kMaxKpt;
  const int i0 = t * kpt;
  const bool vec_ok = !lst && ((reinterpret_cast<uintptr_t>(sc) & 15u) == 0);
  uint32_t k[kMaxKpt];
#pragma unroll
  for (int j4 = 0; j4 < kMaxKpt / 4; ++j4) {
    const int i = i0 + 4 * j4;
    if (4 * j4 < kpt && i + 3 < n && vec_ok) {
      const float4 s4 = *reinterpret_cast<const float4*>(sc + i);
      k[4 * j4 + 0] = order_key(s4.x);
      k[4 * j4 + 1] = order_key(s4.y);
      k[4 * j4 + 2] = order_key(s4.z);
      k[4 * j4 + 3] = order_key(s4.w);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) k[4 * j4 + e] = (4 * j4 < kpt && i + e < n) ? key_global(i + e) : 0u;
    }
  }
  for (int x = t; x < kBins; x += kThreads) hist_s[x] = 0u;
  for (int x = t; x < kRegKeys / 32; x += kThreads) mark_s[x] = 0u;
  if (t == 0) bcount_s = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kMaxKpt; ++j)
    if (k[j] != 0u) atomicAdd(&hist_s[k[j] >> 20], 1u);
  __syncthreads();
  find_bucket(hist_s, kBins, (uint32_t)K, red_s, pick_s, t, lane, wv);  // pick_s[2]: eligible total
  __syncthreads();
  const uint32_t total = pick_s[2];
  const bool take_all = total <= (uint32_t)K;
  const uint32_t bucket = take_all ? 0u : pick_s[0];
  const uint32_t quota = take_all ? 0u : (uint32_t)K - pick_s[1];

  bool ranked = true;  // boundary bucket resolved by direct ranking
  uint32_t thr = 0, take_eq = 0;
  if (!take_all) {
    // gather the boundary bucket: a wave-wide prefix of the per-thread counts
    // and one LDS atomic per wave place every key
    uint32_t nb = 0;
#pragma unroll
    for (int j = 0; j < kMaxKpt; ++j) nb += (k[j] != 0u) & ((k[j] >> 20) == bucket);
    const uint32_t nb_incl = wave_incl_scan(nb);
    uint32_t wbase = 0;
    if (lane == 63 && nb_incl != 0u) wbase = atomicAdd(&bcount_s, nb_incl);
    uint32_t slot = (uint32_t)__builtin_amdgcn_readlane((int)wbase, 63) + nb_incl - nb;
#pragma unroll
    for (int j = 0; j < kMaxKpt; ++j) {
      if (k[j] != 0u && (k[j] >> 20) == bucket) {
        if (slot < (uint32_t)kRankCap) bk_s[slot] = ((uint64_t)k[j] << 32) | (uint32_t)~(uint32_t)(i0 + j);
        ++slot;
      }
    }
    __syncthreads();
    const uint32_t m = bcount_s;
    ranked = m <= (uint32_t)kRankCap;
    if (ranked && m <= (uint32_t)(kThreads / 4)) {
      // four threads per key, each comparing against every fourth key
      const uint32_t key = (uint32_t)t >> 2, part = (uint32_t)t & 3u;
      const uint64_t me = bk_s[key < m ? key : 0u];
      uint32_t r = 0;
      uint32_t q = part;
      for (; q + 28 < m; q += 32) {
        uint64_t o[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) o[u] = bk_s[q + 4 * u];
#pragma unroll
        for (int u = 0; u < 8; ++u) r += (uint32_t)(o[u] > me);
      }
      for (; q < m; q += 4) r += (uint32_t)(bk_s[q] > me);
      // sum the quad (DPP quad_perm [1,0,3,2] then [2,3,0,1])
      r += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)r, 0xB1, 0xf, 0xf, false);
      r += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)r, 0x4E, 0xf, 0xf, false);
      const uint32_t mi = ~(uint32_t)me;
      if (key < m && part == 0u && r < quota) atomicOr(&mark_s[mi >> 5], 1u << (mi & 31));
      __syncthreads();
    } else if (ranked) {
      if ((uint32_t)t < m) {
        // (key desc, index asc) is the unsigned order of key << 32 | ~index
        const uint64_t me = bk_s[t];
        uint32_t r = 0;
        uint32_t q = 0;
        for (; q + 8 <= m; q += 8) {  // eight independent LDS reads in flight
          uint64_t o[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) o[u] = bk_s[q + u];
#pragma unroll
          for (int u = 0; u < 8; ++u) r += (uint32_t)(o[u] > me);
        }
        for (; q < m; ++q) r += (uint32_t)(bk_s[q] > me);
        const uint32_t mi = ~(uint32_t)me;
        if (r < quota) atomicOr(&mark_s[mi >> 5], 1u << (mi & 31));
      }
      __syncthreads();
    } else {
      radix_finish(1, bucket << 20, 0xFFF00000u, quota, hist_s, red_s, pick_s, t, lane, wv,
                   [&](int shift, uint32_t dm, uint32_t prefix, uint32_t pmask) {
#pragma unroll
                     for (int j = 0; j < kMaxKpt; ++j)
                       if (k[j] != 0u && (k[j] & pmask) == prefix) atomicAdd(&hist_s[(k[j] >> shift) & dm], 1u);
                   },
                   thr, take_eq);
    }
  }

  if (ranked) {
    // chosen: eligible (take_all), above the boundary bucket, or a marked bucket key
    bool sel[kMaxKpt];
    uint32_t cnt = 0;
    const uint32_t mword = mark_s[i0 >> 5] >> (i0 & 31);  // this thread's 16 indices share one word
#pragma unroll
    for (int j = 0; j < kMaxKpt; ++j) {
      const uint32_t hb = k[j] >> 20;
      const uint32_t marked = (mword >> j) & 1u;
      sel[j] = take_all ? (k[j] != 0u) : ((hb > bucket) | ((hb == bucket) & (k[j] != 0u) & (marked != 0u)));
      cnt += sel[j];
    }
    uint32_t before, unused, tot_sel, unused2;
    block_prefix2(cnt, 0u, red_s, lane, wv, before, unused, tot_sel, unused2);
#pragma unroll
    for (int j = 0; j < kMaxKpt; ++j) {
      if (sel[j]) {
        if (before < (uint32_t)K) out[before] = row_of(i0 + j);
        ++before;
      }
    }
    pad(tot_sel);
    return;
  }

  // boundary bucket too large to rank: keys above the radix threshold, then the
  // lowest-index keys equal to it
  uint32_t cg = 0, ce = 0;
#pragma unroll
  for (int j = 0; j < kMaxKpt; ++j) {
    cg += (k[j] > thr);
    ce += (k[j] == thr);
  }
  uint32_t gtb, eqb, gt_tot, eq_tot;
  block_prefix2(cg, ce, red_s, lane, wv, gtb, eqb, gt_tot, eq_tot);
#pragma unroll
  for (int j = 0; j < kMaxKpt; ++j) {
    const bool gt = k[j] > thr;
    const bool eq = k[j] == thr;
    if (gt || (eq && eqb < take_eq)) {
      const uint32_t p = gtb + (eqb < take_eq ? eqb : take_eq);
      if (p < (uint32_t)K) out[p] = row_of(i0 + j);
    }
    gtb += gt;
    eqb += eq;
  }
  pad(gt_tot + (eq_tot < take_eq ? eq_tot : take_eq));
}

}  // namespace

hipError_t launch_topk_k(int32_t K, int32_t B, const csa2_batch& bt, const float* scores, int64_t stride,
                         int32_t* topk_idx, hipStream_t s) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(B), dim3(kThreads), 0, s, K, bt.max_candidates, bt.pos, bt.mode,
                     bt.compress_ratio, bt.pool_len, bt.cand_off, bt.cand_idx, scores, stride, topk_idx);
  return hipGetLastError();
}

hipError_t launch_topk(const csa2_dims& d, int32_t B, const csa2_batch& bt, const float* scores,
                       int64_t stride, int32_t* topk_idx, hipStream_t s) {
  return launch_topk_k(d.index_topk, B, bt, scores, stride, topk_idx, s);
}

}  // namespace csa2
