// Top-K selection (Reading Notes of DeepSeek-V4.1-Flash, section 3f C2 Step 2:
// keep the K best-scoring entries; PocketLLM "DeepSeek-V4.1-Flash",
// "Correctness and precision": unused slots hold -1).
//
// Order: score descending, then row ascending (the lowest row wins a tie); +0
// and -0 tie.  Output: the chosen rows in ascending order, then -1s.
//
// One workgroup of NT threads per query.  Scores map to order-preserving
// 32-bit keys; ineligible slots get key 0, below every finite score and -inf.
// The list is read in segments of NT * KPT keys, thread t holding the
// contiguous run [t*KPT, t*KPT+KPT) of a segment in registers; a list of one
// segment stays in registers throughout, a longer one is re-read from the
// score buffer (just written, so from cache) in each pass:
//  1. an LDS histogram of the top 12 key bits and a block-wide suffix scan
//     find the bucket that holds the K-th best key and how many keys lie above
//     it (and the eligible total: at most K eligible means take them all);
//  2. the keys of that bucket (typically 1-2 % of them) are gathered into LDS
//     with their indices and ranked exactly against each other under
//     (key desc, index asc); the one ranked at the remaining quota is the K-th
//     key overall, (th, idx_lim);
//  3. compaction: a key is chosen iff key > th, or key == th and its index is
//     <= idx_lim; a block-wide prefix over threads (= index order) of the
//     per-thread counts, carried across segments, places every chosen row.
// When the boundary bucket is too large to rank (heavy ties), a radix select
// over the two remaining digits (bits 19-8, 7-0) finds the K-th key value and
// a prefix over the keys equal to it finds its index.
//
// The forms (launch_forms picks one per batch):
//  - the survivor form (topk_lean_kernel, below) for batches of 512 queries
//    or more whose lists fit one 512 x 32 segment and carry no Reindex list:
//    a floor from the threads' largest keys leaves ~18 % of the keys, and
//    every pass after the first runs over those survivors only; three
//    workgroups per CU hide each other's barrier and LDS waits;
//  - the register-segment form above (topk_run), 512 threads x 32 keys, for
//    the same lists in smaller batches (one workgroup alone on a CU: its
//    shorter chain of passes has the lower latency);
//  - 1,024 x 16 (few queries) and 512 x 32 (many queries) general shapes for
//    longer lists and Reindex lists, segments re-read per pass; with a
//    workspace, a few long lists split over workgroups (kSegment) and merge
//    in a 512 x 4 / 512 x 8 shape.
#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int kBins = 4096;

__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;  // -0 ties with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

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
template <int kWaves>
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
template <int kWaves>
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

// Find the bucket of an nb-bucket histogram that holds the krem-th largest
// key: each thread owns a run of consecutive buckets, a block-wide suffix scan
// gives the count above each run.  pick_s[0] = bucket, pick_s[1] = keys above
// it, pick_s[2] = all keys counted, pick_s[3] = keys in the bucket.  Contains
// barriers; call uniformly.
template <int kThreads>
__device__ __forceinline__ void find_bucket(const uint32_t* hist_s, int nb, uint32_t krem, uint32_t* red_s,
                                            uint32_t* pick_s, int t, int lane, int wv) {
  constexpr int kMaxBpt = kBins / kThreads;  // histogram buckets owned per thread (>= 1)
  const int bpt = (nb + kThreads - 1) / kThreads;
  uint32_t c[kMaxBpt], tot = 0;
#pragma unroll
  for (int u = 0; u < kMaxBpt; ++u) {
    const int bkt = t * bpt + u;
    c[u] = (u < bpt && bkt < nb) ? hist_s[bkt] : 0u;
    tot += c[u];
  }
  uint32_t above = block_suffix_excl<kThreads / 64>(tot, red_s, lane, wv);
  if (t == 0) pick_s[2] = above + tot;
#pragma unroll
  for (int u = kMaxBpt - 1; u >= 0; --u) {
    if (u < bpt) {
      if (above < krem && krem <= above + c[u]) {
        pick_s[0] = t * bpt + u;
        pick_s[1] = above;
        pick_s[3] = c[u];
      }
      above += c[u];
    }
  }
}

// Radix select over digits d0 .. 2 (bits 31-20, 19-8, 7-0) starting from a
// known prefix; `count_keys(shift, nb, prefix, pmask)` adds the keys matching
// the prefix into hist_s.  Returns the K-th key and the quota left among keys
// equal to it.
template <int kThreads, typename CountFn>
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
    find_bucket<kThreads>(hist_s, nb, krem, red_s, pick_s, t, lane, wv);
    __syncthreads();
    krem -= pick_s[1];
    prefix |= pick_s[0] << shift;
    pmask |= dm << shift;
    __syncthreads();
  }
  thr = prefix;
  take_eq = krem;
}

// Rank the m (<= kRankCap) keys gathered in bk_s against each other under the
// unsigned order of (key << 32 | ~index); the one ranked quota - 1 (0-based)
// is written to *thr_s.  Keys are distinct (their indices differ), so exactly
// one thread writes.
template <int kThreads>
__device__ __forceinline__ void rank_bucket(const uint64_t* bk_s, uint32_t m, uint32_t quota, uint64_t* thr_s,
                                            int t) {
  // rank the bucket's keys against each other; the one ranked quota-1
  // is the K-th key overall
  if (m <= (uint32_t)(kThreads / 4)) {
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
    if (key < m && part == 0u && r == quota - 1u) *thr_s = me;
  } else if (m <= (uint32_t)(kThreads / 2)) {
    // two threads per key (the usual bucket of a 16,384-key list holds
    // ~200), each comparing against every other key
    const uint32_t key = (uint32_t)t >> 1, part = (uint32_t)t & 1u;
    const uint64_t me = bk_s[key < m ? key : 0u];
    uint32_t r = 0;
    uint32_t q = part;
    for (; q + 14 < m; q += 16) {
      uint64_t o[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) o[u] = bk_s[q + 2 * u];
#pragma unroll
      for (int u = 0; u < 8; ++u) r += (uint32_t)(o[u] > me);
    }
    for (; q < m; q += 2) r += (uint32_t)(bk_s[q] > me);
    // sum the pair (DPP quad_perm [1,0,3,2])
    r += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)r, 0xB1, 0xf, 0xf, false);
    if (key < m && part == 0u && r == quota - 1u) *thr_s = me;
  } else {
    // one thread per key, several keys per thread past kThreads
    for (uint32_t key = (uint32_t)t; key < m; key += kThreads) {
      // (key desc, index asc) is the unsigned order of key << 32 | ~index
      const uint64_t me = bk_s[key];
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
      if (r == quota - 1u) *thr_s = me;
    }
  }
}

// Forms of the kernel:
//   kGeneral  any list, re-read in segments when it outgrows the registers;
//   kOneSeg   every list fits one segment and none is a Reindex list (the
//             launcher's choice): keys loaded once, the re-reading paths gone
//             with their registers;
//   kSegment  workgroup (b, s) takes segment s of query b's list as its list
//             (one register segment, Reindex lists included) and writes its
//             own top-K, rows and scores, to the split buffers, padded with
//             -1; a second pass (kGeneral over those as Reindex lists) picks
//             the query's top-K from them.  Exact: under the strict
//             (score, row) order the K best of a list are among the K best of
//             the segments holding them.
constexpr int kGeneral = 0, kOneSeg = 1, kSegment = 2;
struct TopkSplit {
  int32_t nseg;        // segments per query (kSegment)
  int32_t* rows;       // [B][nseg][K]: each segment's chosen rows, ascending, -1 padded
  float* scores;       // [B][nseg][K]: their scores
  int32_t* mode2;      // [B]: Reindex for a query that selects, else its own mode
  int64_t* off2;       // [B + 1]: b * nseg * K
};

// The LDS a workgroup of topk_run works in (the caller owns it, so another
// kernel can run topk_run over storage it also uses for other purposes).
struct TopkLds {
  uint32_t* hist;    // [kBins], 16-byte aligned
  uint32_t* red;     // [2 * waves]
  uint32_t* pick;    // [4]
  uint64_t* bk;      // [kRankCap]: boundary-bucket (key << 32 | ~index)
  uint64_t* thr;     // the K-th key, (key << 32 | ~index)
  uint32_t* bcount;  // boundary keys gathered
};

template <int kThreads, int kKpt, int kForm>
__device__ __forceinline__ void topk_run(int32_t K, int32_t max_cand, const int64_t* __restrict__ pos,
                                         const int32_t* __restrict__ mode, const int32_t* __restrict__ ratio,
                                         const int32_t* __restrict__ pool_len, const int64_t* __restrict__ cand_off,
                                         const int32_t* __restrict__ cand_idx, const float* __restrict__ scores,
                                         int64_t stride, int32_t* __restrict__ topk_idx, TopkSplit split,
                                         const TopkLds& L) {
  constexpr bool kOne = kForm != kGeneral;  // the list is one register segment
  constexpr int kWaves = kThreads / 64;
  constexpr int kSeg = kThreads * kKpt;  // keys per segment (one key register set)
  static_assert(kKpt % 4 == 0, "keys are loaded four at a time");
  // A thread's per-key decisions are kept as bits of one 32-bit mask (one
  // register) between counting and placing, rather than as kKpt condition
  // masks held across the block-wide scan in between.
  static_assert(kKpt <= 32, "a thread's keys fit one bit mask");
  uint32_t* const hist_s = L.hist;
  uint32_t* const red_s = L.red;
  uint32_t* const pick_s = L.pick;
  uint64_t* const bk_s = L.bk;
  uint64_t& thr_s = *L.thr;
  uint32_t& bcount_s = *L.bcount;

  // queries in reverse: a batch's scores are written in query order just
  // before, so the last rows written, the likeliest to be in the last-level
  // cache, are read first (forward, the first misses evict them)
  const int b = kForm == kSegment ? (int)blockIdx.x : (int)gridDim.x - 1 - (int)blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const int md = mode[b];
  if constexpr (kForm == kSegment) {
    if (blockIdx.y == 0 && t == 0) {
      split.mode2[b] = (md == CSA2_MODE_FULL || md == CSA2_MODE_REINDEX) ? CSA2_MODE_REINDEX : md;
      split.off2[b] = (int64_t)b * split.nseg * K;
      if (b == (int)gridDim.x - 1) split.off2[b + 1] = (int64_t)(b + 1) * split.nseg * K;
    }
  }
  if (md != CSA2_MODE_FULL && md != CSA2_MODE_REINDEX) return;
  const int64_t nv = n_valid_of(pos[b], ratio[b], md, pool_len[b]);
  // a REINDEX query without lists (cand_off NULL) has an empty list
  int64_t n64 = (md == CSA2_MODE_FULL) ? nv : (cand_off ? cand_off[b + 1] - cand_off[b] : 0);
  if (n64 > max_cand) n64 = max_cand;
  // kSegment: this workgroup's part of the list, positions first .. first + n - 1
  const int64_t first = kForm == kSegment ? (int64_t)blockIdx.y * (kThreads * kKpt) : 0;
  if (kForm == kSegment) n64 = n64 > first ? (n64 - first < kThreads * kKpt ? n64 - first : kThreads * kKpt) : 0;
  const int n = (int)n64;
  const int32_t* lst =
      (kForm != kOneSeg && md == CSA2_MODE_REINDEX && n64 > 0) ? cand_idx + cand_off[b] + first : nullptr;
  const float* sc = scores + (int64_t)b * stride + first;
  int32_t* out = kForm == kSegment ? split.rows + ((int64_t)b * split.nseg + blockIdx.y) * K
                                   : topk_idx + (int64_t)b * K;
  const bool sc_aligned = (reinterpret_cast<uintptr_t>(sc) & 15u) == 0;
  auto pad = [&](uint32_t chosen) {
    if (chosen > (uint32_t)K) chosen = K;
    for (int x = (int)chosen + t; x < K; x += kThreads) out[x] = -1;
  };

  // Thread t holds keys s*kSeg + t*kKpt + j, j < kKpt, of segment s.  Bounds
  // are tested as j < nrem with j a constant, so no per-key index stays live.
  const int nseg = kOne ? 1 : (n + kSeg - 1) / kSeg;
  uint32_t k[kKpt];
  auto load_seg = [&](int s) __attribute__((always_inline)) {
    const int base = s * kSeg + t * kKpt;
    const int nrem = n - base;
    const float* sp = sc + base;
    if (nrem >= kKpt && sc_aligned) {
      const float4* p4 = reinterpret_cast<const float4*>(sp);
#pragma unroll
      for (int j4 = 0; j4 < kKpt / 4; ++j4) {
        const float4 s4 = p4[j4];
        k[4 * j4 + 0] = order_key(s4.x);
        k[4 * j4 + 1] = order_key(s4.y);
        k[4 * j4 + 2] = order_key(s4.z);
        k[4 * j4 + 3] = order_key(s4.w);
      }
    } else {
      // the thread that straddles the list's end (or an unaligned row):
      // whole float4s while they lie inside the list, single keys after
      // (32 single loads in one lane would hold its wave, and the
      // workgroup's next barrier, for thousands of cycles)
#pragma unroll
      for (int j4 = 0; j4 < kKpt / 4; ++j4) {
        if (sc_aligned && 4 * j4 + 4 <= nrem) {
          const float4 s4 = reinterpret_cast<const float4*>(sp)[j4];
          k[4 * j4 + 0] = order_key(s4.x);
          k[4 * j4 + 1] = order_key(s4.y);
          k[4 * j4 + 2] = order_key(s4.z);
          k[4 * j4 + 3] = order_key(s4.w);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) k[4 * j4 + q] = (4 * j4 + q < nrem) ? order_key(sp[4 * j4 + q]) : 0u;
        }
      }
    }
    if (kForm != kOneSeg && lst) {  // REINDEX rows outside the reachable range are ineligible
      const int32_t* lp = lst + base;
#pragma unroll
      for (int j = 0; j < kKpt; ++j) {
        if (j < nrem) {
          const int32_t r = lp[j];
          if (r < 0 || r >= nv) k[j] = 0u;
        }
      }
    }
  };
  // one segment: its keys stay in registers through every pass
  if (nseg == 1) load_seg(0);
  auto seg_keys = [&](int s) __attribute__((always_inline)) {
    if (!kOne && nseg > 1) load_seg(s);
  };

  // ---- pass 1: histogram of the eligible keys ----
  // A floor below which no chosen key lies: the largest keys of the P
  // threads that hold keys are P distinct keys, and the second largest of
  // the first K - P of them (when P < K; a list a little short of the
  // segment leaves its last threads empty) K - P more, so at least K keys
  // are >= the smallest of those, and so is the K-th best.  Keys below it
  // are set ineligible (0) before counting: for Gaussian scores about a
  // sixth of the list stays.
  // The histogram then spans the survivors' own range, [floor, largest key]
  // in 4,096 bins of 2^shift keys, so the boundary bin of a 16,384-key list
  // holds a key or two rather than the ~200 that bins of the top 12 key bits
  // hold there (the ranking and the gather that follow scale with it), and
  // the counting atomics rarely meet on one bin.  Only for a list held in
  // registers (one segment); otherwise the bins are the top 12 key bits.  The
  // waves' minima and maxima travel with the barrier that clears the
  // histogram.
  const bool floored = nseg == 1 && K <= kThreads;
  for (int x = t; x < kBins / 4; x += kThreads) reinterpret_cast<uint4*>(hist_s)[x] = make_uint4(0u, 0u, 0u, 0u);
  if (t == 0) bcount_s = 0u;
  if (floored) {
    uint32_t m = 0u, m2 = 0u;  // the thread's largest and second largest keys
#pragma unroll
    for (int j = 0; j < kKpt; ++j) {
      const uint32_t lo2 = k[j] < m ? k[j] : m;
      m2 = lo2 > m2 ? lo2 : m2;
      m = k[j] > m ? k[j] : m;
    }
    uint32_t mx = m;
    const int P = (n + kKpt - 1) / kKpt < kThreads ? (n + kKpt - 1) / kKpt : kThreads;  // threads holding keys
    const int D = K > P ? K - P : 0;
    // D > P: too short a list for a floor (0 keeps every key)
    m = D > P ? 0u : (t < D ? m2 : (t < P ? m : 0xFFFFFFFFu));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)m, off, 64);
      const uint32_t ox = (uint32_t)__shfl_xor((int)mx, off, 64);
      m = o < m ? o : m;
      mx = ox > mx ? ox : mx;
    }
    if (lane == 0) red_s[wv] = m, red_s[kWaves + wv] = mx;
  }
  __syncthreads();
  uint32_t kbase = 0u;  // bin of an eligible key: (key - kbase) >> kshift
  int kshift = 20;
  if (floored) {
    uint32_t floor = red_s[0], top = red_s[kWaves];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      floor = red_s[w] < floor ? red_s[w] : floor;
      top = red_s[kWaves + w] > top ? red_s[kWaves + w] : top;
    }
#pragma unroll
    for (int j = 0; j < kKpt; ++j) k[j] = k[j] >= floor ? k[j] : 0u;
    kbase = floor > 1u ? floor : 1u;  // eligible keys are >= 1
    const uint32_t range = top > kbase ? top - kbase : 0u;
    const int bits = range ? 32 - __clz((int)range) : 0;
    kshift = bits > 12 ? bits - 12 : 0;  // range >> kshift < 4,096
  }
  for (int s = 0; s < nseg; ++s) {
    seg_keys(s);
#pragma unroll
    for (int j = 0; j < kKpt; ++j)
      if (k[j] != 0u) atomicAdd(&hist_s[(k[j] - kbase) >> kshift], 1u);
  }
  __syncthreads();  // (also orders the floor's reads of red_s before find_bucket writes it)
  find_bucket<kThreads>(hist_s, kBins, (uint32_t)K, red_s, pick_s, t, lane, wv);  // pick_s[2]: eligible total
  __syncthreads();
  const uint32_t total = pick_s[2];
  const bool take_all = total <= (uint32_t)K;

  // The chosen keys are exactly those with (key << 32 | ~index) >= that of
  // the K-th best key; with the K-th key as (th, idx_lim) a key is chosen iff
  // key > th, or key == th and index <= idx_lim.
  uint32_t th = 1u;              // take_all: every eligible key (key >= 1)
  int32_t idx_lim = 0x7fffffff;
  if (!take_all) {
    const uint32_t bucket = pick_s[0];
    const uint32_t quota = (uint32_t)K - pick_s[1];  // 1 .. keys in the bucket
    const uint32_t lo = kbase + (bucket << kshift), width = 1u << kshift;  // the bucket: keys lo .. lo + width - 1
    // ---- pass 2: gather the boundary bucket (a wave-wide prefix of the
    // per-thread counts and one LDS atomic per wave place every key) ----
    for (int s = 0; s < nseg; ++s) {
      seg_keys(s);
      uint32_t bm = 0;  // keys of the boundary bucket
#pragma unroll
      for (int j = 0; j < kKpt; ++j) bm |= (uint32_t)((k[j] != 0u) & ((k[j] - lo) < width)) << j;
      const uint32_t nb = (uint32_t)__popc(bm);
      const uint32_t nb_incl = wave_incl_scan(nb);
      uint32_t wbase = 0;
      if (lane == 63 && nb_incl != 0u) wbase = atomicAdd(&bcount_s, nb_incl);
      uint32_t slot = (uint32_t)__builtin_amdgcn_readlane((int)wbase, 63) + nb_incl - nb;
      const uint32_t gbase = (uint32_t)(s * kSeg + t * kKpt);
      // over the set bits only (a thread holds a key or two of the bucket;
      // a branch per key position would cost every wave all kKpt of them);
      // the key at a dynamic position comes from its register by a select
      // chain, kept off the common path
      for (uint32_t rest = bm; rest != 0u; rest &= rest - 1u) {
        const int j = __builtin_ctz(rest);
        uint32_t kj = 0u;
#pragma unroll
        for (int q = 0; q < kKpt; ++q) kj = q == j ? k[q] : kj;
        if (slot < (uint32_t)kRankCap) bk_s[slot] = ((uint64_t)kj << 32) | (uint32_t)~(gbase + (uint32_t)j);
        ++slot;
      }
    }
    __syncthreads();
    const uint32_t m = bcount_s;
    if (m <= (uint32_t)kRankCap) {
      rank_bucket<kThreads>(bk_s, m, quota, &thr_s, t);
    } else {
      // heavy ties: radix select over the bucket's keys gives the K-th key
      // value and how many keys equal to it are taken (lowest indices
      // first); the last of those, found by a prefix over the keys in index
      // order, is the K-th key.  This rare path re-reads the keys, so the
      // register copy need not stay live through it.
      uint32_t thr = 0, take_eq = 0;
      radix_finish<kThreads>(0, 0u, 0u, quota, hist_s, red_s, pick_s, t, lane, wv,
                             [&](int shift, uint32_t dm, uint32_t prefix, uint32_t pmask) __attribute__((always_inline)) {
                               for (int s = 0; s < nseg; ++s) {
                                 if (!kOne) load_seg(s);
#pragma unroll
                                 for (int j = 0; j < kKpt; ++j)
                                   if (k[j] != 0u && (k[j] - lo) < width && (k[j] & pmask) == prefix)
                                     atomicAdd(&hist_s[(k[j] >> shift) & dm], 1u);
                               }
                             },
                             thr, take_eq);
      uint32_t carry = 0;
      for (int s = 0; s < nseg; ++s) {
        if (!kOne) load_seg(s);
        uint32_t em = 0;  // keys equal to the K-th value
#pragma unroll
        for (int j = 0; j < kKpt; ++j) em |= (uint32_t)(k[j] == thr) << j;
        const uint32_t ce = (uint32_t)__popc(em);
        uint32_t before, unused, tot_eq, unused2;
        block_prefix2<kWaves>(ce, 0u, red_s, lane, wv, before, unused, tot_eq, unused2);
        before += carry;
        if (before < take_eq && take_eq <= before + ce) {
          const uint32_t gbase = (uint32_t)(s * kSeg + t * kKpt);
#pragma unroll
          for (int j = 0; j < kKpt; ++j) {
            if ((em >> j) & 1u) {
              if (++before == take_eq) thr_s = ((uint64_t)thr << 32) | (uint32_t)~(gbase + j);
            }
          }
        }
        carry += tot_eq;
        __syncthreads();
      }
    }
    __syncthreads();
    const uint64_t kth = thr_s;
    th = (uint32_t)(kth >> 32);
    idx_lim = (int32_t)~(uint32_t)kth;
  }

  // ---- pass 3: compaction in index order (a block-wide prefix of the
  // per-thread counts, carried from segment to segment).  With K up to the
  // histogram's size the chosen rows are placed in the (now free) histogram
  // first and written out with one coalesced pass, -1 padded ----
  const bool staged = K <= kBins;
  uint32_t carry = 0;
  for (int s = 0; s < nseg; ++s) {
    seg_keys(s);
    const int base = s * kSeg + t * kKpt;
    const int jl = idx_lim - base;  // key j of this thread may equal th iff j <= jl
    uint32_t cm = 0;  // chosen keys
#pragma unroll
    for (int j = 0; j < kKpt; ++j) cm |= (uint32_t)((k[j] > th) | ((k[j] == th) & (j <= jl))) << j;
    const uint32_t cnt = (uint32_t)__popc(cm);
    uint32_t before, unused, tot_sel, unused2;
    block_prefix2<kWaves>(cnt, 0u, red_s, lane, wv, before, unused, tot_sel, unused2);
    before += carry;
    {
      // over the set bits only (about one chosen key per thread)
      const int32_t* lp = (kForm != kOneSeg && lst) ? lst + base : nullptr;
      const uint32_t lim = before < (uint32_t)K ? (uint32_t)K - before : 0u;  // places left
      uint32_t rest = cnt > lim ? 0u : cm;
      if (cnt > lim)  // the last places: the chosen keys of lowest position
        for (uint32_t r = cm, c = 0; c < lim; ++c, r &= r - 1u) rest |= r & (0u - r);
      for (; rest != 0u; rest &= rest - 1u) {
        const int j = __builtin_ctz(rest);
        // kSegment stages the list position (its row and score are both read out below)
        const int32_t row = kForm == kSegment ? base + j : (lp ? lp[j] : base + j);
        if (staged) hist_s[before] = (uint32_t)row;
        else out[before] = row;
        ++before;
      }
    }
    carry += tot_sel;
    __syncthreads();
  }
  if constexpr (kForm == kSegment) {  // K <= kBins here (the launcher's choice)
    const uint32_t n_out = carry < (uint32_t)K ? carry : (uint32_t)K;
    float* so = split.scores + ((int64_t)b * split.nseg + blockIdx.y) * K;
    for (int x = t; x < K; x += kThreads) {
      const bool has = (uint32_t)x < n_out;
      const int32_t p = has ? (int32_t)hist_s[x] : 0;
      out[x] = has ? (lst ? lst[p] : (int32_t)(first + p)) : -1;
      so[x] = has ? sc[p] : -__builtin_inff();
    }
  } else if (staged) {
    const uint32_t n_out = carry < (uint32_t)K ? carry : (uint32_t)K;
    for (int x = t; x < K; x += kThreads) out[x] = (uint32_t)x < n_out ? (int32_t)hist_s[x] : -1;
  } else {
    pad(carry);
  }
}

template <int kThreads, int kKpt, int kForm>
__global__ __launch_bounds__(kThreads, kThreads == 512 ? 4 : 1) void topk_kernel(
    int32_t K, int32_t max_cand, const int64_t* __restrict__ pos, const int32_t* __restrict__ mode,
    const int32_t* __restrict__ ratio, const int32_t* __restrict__ pool_len,
    const int64_t* __restrict__ cand_off, const int32_t* __restrict__ cand_idx,
    const float* __restrict__ scores, int64_t stride, int32_t* __restrict__ topk_idx, TopkSplit split) {
  __shared__ __attribute__((aligned(16))) uint32_t hist_s[kBins];
  __shared__ uint32_t red_s[2 * (kThreads / 64)];
  __shared__ uint32_t pick_s[4];
  __shared__ uint64_t bk_s[kRankCap];
  __shared__ uint64_t thr_s;
  __shared__ uint32_t bcount_s;
  const TopkLds L{hist_s, red_s, pick_s, bk_s, &thr_s, &bcount_s};
  topk_run<kThreads, kKpt, kForm>(K, max_cand, pos, mode, ratio, pool_len, cand_off, cand_idx, scores, stride,
                                  topk_idx, split, L);
}

// ---------------------------------------------------------------------------
// The survivor form: one workgroup of 512 threads per query for lists of
// 2,048 .. 16,384 candidates (no Reindex lists, K <= 512), launched for
// batches of 512 queries or more.
//
// The list is read as 8 chunks of 2,048 keys, thread t holding keys
// 2048c + 4t .. 2048c + 4t + 3 of chunk c (one 16-byte load per chunk, so
// each load instruction of a wave reads 1 KiB of consecutive scores).  Every
// thread holds at least one key of the first chunk, so the 512 threads'
// largest keys are 512 >= K distinct keys, and the smallest of them is a
// floor: no key below it can be among the K best.
//
// With a positive floor, the order of keys at or above it is the order of
// the scores' bit patterns read as signed integers (non-negative patterns are
// the positive scores, +inf and +NaN patterns above them in the same order the
// key map gives them; every pattern with the sign bit set, -0 included, maps
// below +0 and so below the floor).  The floor test is one integer compare
// per key, with no key map at all.  Keys at or above the floor (for Gaussian
// scores about 18 % of the list: the floor is the smallest of 512 maxima of
// 32) are appended to their wave's survivor list in LDS (score bits and
// ~position) by a wave-wide ballot and prefix.  Every later pass runs over
// the survivors only, a few per lane instead of 32 keys per thread:
//  1. a 4,096-bin histogram over [floor, largest key] finds the bucket that
//     holds the K-th best survivor and how many lie above it;
//  2. when that bucket holds exactly the survivors still needed (usually
//     one), all of it is chosen; otherwise its survivors are ranked exactly
//     under (score desc, position asc): the K-th key (th, index limit);
//  3. each chosen survivor sets its position's bit in a 16,384-bit LDS map;
//     thread t owns word t (positions 32t .. 32t + 31), so a block-wide
//     prefix over the words' popcounts writes the chosen rows in ascending
//     order.
// Whatever this form does not cover goes through the register-segment form
// (topk_run, kOneSeg) on the same LDS: a short or unaligned list, a floor at
// or below +0 (some thread holds no positive score), a wave with more than
// kLCap survivors, or a boundary bucket of more than kRankCap keys (heavy
// ties).  The results are the same either way.
constexpr int kLThreads = 512, kLWaves = kLThreads / 64;
constexpr int kLChunks = 8, kLSpan = kLThreads * 4;  // 2,048 keys per chunk
constexpr int kLMax = kLChunks * kLSpan;               // 16,384
constexpr uint32_t kLCap = 512;                        // survivors a wave's list holds
constexpr uint32_t kLPos = kLWaves * kLCap;            // from a survivor's bits to its ~position

__global__ __launch_bounds__(kLThreads) __attribute__((amdgpu_waves_per_eu(6))) void topk_lean_kernel(
    int32_t K, int32_t max_cand, const int64_t* __restrict__ pos, const int32_t* __restrict__ mode,
    const int32_t* __restrict__ ratio, const int32_t* __restrict__ pool_len,
    const int64_t* __restrict__ cand_off, const int32_t* __restrict__ cand_idx,
    const float* __restrict__ scores, int64_t stride, int32_t* __restrict__ topk_idx, TopkSplit split) {
  __shared__ __attribute__((aligned(16))) uint32_t hist_s[kBins];
  // survivors: wave w's score bits at [w kLCap, ..), their ~positions kLPos
  // words further on; the fallback's bk list
  __shared__ __attribute__((aligned(16))) uint32_t surv_s[2 * kLWaves * kLCap];
  __shared__ uint32_t map_s[kLThreads];  // chosen positions, one bit each
  __shared__ uint32_t red_s[2 * kLWaves];
  __shared__ uint32_t pick_s[4];
  __shared__ uint32_t cnt_s[kLWaves];
  __shared__ uint64_t thr_s;
  __shared__ uint32_t bcount_s;
  static_assert(2 * kLWaves * kLCap * 4 >= kRankCap * 8, "the fallback's bk list fits the survivor lists");
  const TopkLds L{hist_s, red_s, pick_s, reinterpret_cast<uint64_t*>(surv_s), &thr_s, &bcount_s};
  // the survivor path; false: the query goes through topk_run instead (a
  // uniform decision, taken before or after a barrier; one call site keeps
  // one inlined copy of topk_run)
  auto survivors = [&]() __attribute__((always_inline)) -> bool {
  const int b = (int)gridDim.x - 1 - (int)blockIdx.x;  // queries in reverse, as in topk_run
  const int t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const int md = mode[b];
  if (md != CSA2_MODE_FULL && md != CSA2_MODE_REINDEX) return true;
  int64_t n64 = md == CSA2_MODE_FULL ? n_valid_of(pos[b], ratio[b], md, pool_len[b]) : 0;
  if (n64 > max_cand) n64 = max_cand;
  const float* sc = scores + (int64_t)b * stride;
  if (cand_off != nullptr || K < 1 || K > kLThreads || n64 < kLSpan || n64 > kLMax ||
      (reinterpret_cast<uintptr_t>(sc) & 15u) != 0)
    return false;
  const int n = (int)n64;
  int32_t* out = topk_idx + (int64_t)b * K;

  // ---- the keys (score bits as signed integers), the thread's largest ----
  int v[kLChunks * 4];
#pragma unroll
  for (int c = 0; c < kLChunks; ++c) {
    // positions past the list's end are INT32_MIN, below any positive floor;
    // only the thread that straddles the end loads single scores
    const int off = c * kLSpan + 4 * t;
    int4 x = make_int4(INT32_MIN, INT32_MIN, INT32_MIN, INT32_MIN);
    if (off + 4 <= n) {
      x = reinterpret_cast<const int4*>(sc + off)[0];
    } else if (off < n) {
      x.x = __float_as_int(sc[off]);
      if (off + 1 < n) x.y = __float_as_int(sc[off + 1]);
      if (off + 2 < n) x.z = __float_as_int(sc[off + 2]);
    }
    v[4 * c + 0] = x.x, v[4 * c + 1] = x.y, v[4 * c + 2] = x.z, v[4 * c + 3] = x.w;
  }
  int mx = v[0];
#pragma unroll
  for (int j = 1; j < kLChunks * 4; ++j) mx = v[j] > mx ? v[j] : mx;
  int lo_m = mx, hi_m = mx;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const int a = __shfl_xor(lo_m, off, 64), c = __shfl_xor(hi_m, off, 64);
    lo_m = a < lo_m ? a : lo_m;
    hi_m = c > hi_m ? c : hi_m;
  }
  for (int x = t; x < kBins / 4; x += kLThreads) reinterpret_cast<uint4*>(hist_s)[x] = make_uint4(0u, 0u, 0u, 0u);
  map_s[t] = 0u;
  if (t == 0) bcount_s = 0u;
  if (lane == 0) red_s[wv] = (uint32_t)lo_m, red_s[kLWaves + wv] = (uint32_t)hi_m;
  __syncthreads();
  // the block's floor and largest key, reduced over eight lanes and kept
  // wave-uniform (scalar registers)
  int fl = lane < kLWaves ? (int)red_s[lane] : INT32_MAX;
  int tp = lane < kLWaves ? (int)red_s[kLWaves + lane] : INT32_MIN;
#pragma unroll
  for (int off = 4; off >= 1; off >>= 1) {
    const int a = __shfl_xor(fl, off, 64), c = __shfl_xor(tp, off, 64);
    fl = a < fl ? a : fl;
    tp = c > tp ? c : tp;
  }
  const int floor = __builtin_amdgcn_readfirstlane(fl), top = __builtin_amdgcn_readfirstlane(tp);
  if (floor < 1) return false;  // a thread without a positive score: no integer floor
  const uint32_t range = (uint32_t)(top - floor);
  const int rbits = range ? 32 - __clz((int)range) : 0;
  const int kshift = rbits > 12 ? rbits - 12 : 0;  // range >> kshift < 4,096

  // ---- survivors: keys >= floor, appended to the wave's list ----
  // (the list's base and count are wave-uniform scalars, so a survivor's
  // address is one shift-add of its lane's ballot prefix, and its bits and
  // ~position go out as two 4-byte writes at a constant distance)
  uint32_t* const mine = surv_s + kLCap * (uint32_t)__builtin_amdgcn_readfirstlane(wv);
  const uint32_t npos = ~(uint32_t)(4 * t);  // ~position of the thread's first key of chunk 0
  uint32_t wcnt = 0;                          // the wave's survivors so far (wave-uniform)
#pragma unroll
  for (int j = 0; j < kLChunks * 4; ++j) {
    const bool e = v[j] >= floor;
    const uint64_t bal = __ballot(e);
    const uint32_t nb = (uint32_t)__popcll(bal);
    if (wcnt + nb <= kLCap && e) {
      const uint32_t pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      uint32_t* const at = mine + wcnt + pre;
      at[0] = (uint32_t)v[j];
      at[kLPos] = npos ^ (uint32_t)((j >> 2) * kLSpan + (j & 3));  // ~position (the bits are disjoint)
    }
    wcnt += nb;
  }
  // this wave's histogram (its own list: no barrier, only the wave's own
  // LDS writes to see)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint32_t nsurv = wcnt < kLCap ? wcnt : kLCap;
  for (uint32_t i = (uint32_t)lane; i < nsurv; i += 64)
    atomicAdd(&hist_s[(mine[i] - (uint32_t)floor) >> kshift], 1u);
  if (lane == 0) cnt_s[wv] = wcnt;
  __syncthreads();
  bool ovf = false;
#pragma unroll
  for (int w = 0; w < kLWaves; ++w) ovf |= cnt_s[w] > kLCap;
  if (ovf) return false;
  find_bucket<kLThreads>(hist_s, kBins, (uint32_t)K, red_s, pick_s, t, lane, wv);  // pick_s[2]: survivors
  __syncthreads();
  const uint32_t total = pick_s[2];

  // a survivor is chosen iff bits > th, or bits == th and position <= plim
  uint32_t th = 0u, plim = 0xFFFFFFFFu;  // every survivor (its bits are >= floor >= 1)
  const uint32_t bucket = pick_s[0];
  const uint32_t quota = (uint32_t)K - pick_s[1];  // 1 .. survivors in the bucket
  const uint32_t lo = (uint32_t)floor + (bucket << kshift), width = 1u << kshift;
  if (total > (uint32_t)K && pick_s[3] == quota) {
    // the bucket's survivors are all chosen (usually the bucket holds just
    // the one survivor still needed): the chosen ones are those >= lo, and
    // there is nothing to rank
    th = lo;
  } else if (total > (uint32_t)K) {
    // the bucket's survivors into bk (the histogram's storage, read for the
    // last time by find_bucket before the barrier above)
    uint64_t* const bk = reinterpret_cast<uint64_t*>(hist_s);
    for (uint32_t i0 = 0; i0 < nsurv; i0 += 64) {
      const uint32_t i = i0 + (uint32_t)lane;
      const bool in = i < nsurv;
      const uint32_t kb = in ? mine[i] : 0u;
      const bool isb = in && (kb - lo) < width;
      const uint64_t bal = __ballot(isb);
      if (bal != 0u) {
        uint32_t base = 0u;
        if (lane == 0) base = atomicAdd(&bcount_s, (uint32_t)__popcll(bal));
        base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
        const uint32_t slot =
            __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, base));
        if (isb && slot < (uint32_t)kRankCap) bk[slot] = ((uint64_t)kb << 32) | mine[i + kLPos];
      }
    }
    __syncthreads();
    const uint32_t m = bcount_s;
    if (m > (uint32_t)kRankCap) return false;  // heavy ties
    rank_bucket<kLThreads>(bk, m, quota, &thr_s, t);
    __syncthreads();
    const uint64_t kth = thr_s;
    th = (uint32_t)(kth >> 32);
    plim = ~(uint32_t)kth;
  }

  // ---- the chosen survivors' bits, then rows in ascending order ----
  for (uint32_t i = (uint32_t)lane; i < nsurv; i += 64) {
    const uint32_t kb = mine[i], p = ~mine[i + kLPos];
    if (kb > th || (kb == th && p <= plim)) atomicOr(&map_s[p >> 5], 1u << (p & 31u));
  }
  __syncthreads();
  const uint32_t word = map_s[t];
  uint32_t before, unused, n_out, unused2;
  block_prefix2<kLWaves>((uint32_t)__popc(word), 0u, red_s, lane, wv, before, unused, n_out, unused2);
  // stage the rows (hist_s is free again: bk's last reads were before the
  // barrier above) and write them out in one coalesced pass, -1 padded
  for (uint32_t rest = word; rest != 0u; rest &= rest - 1u) hist_s[before++] = 32u * (uint32_t)t + __builtin_ctz(rest);
  __syncthreads();
  for (int x = t; x < K; x += kLThreads) out[x] = (uint32_t)x < n_out ? (int32_t)hist_s[x] : -1;
  return true;
  };
  if (survivors()) return;
  __syncthreads();  // the survivor path's LDS reads are done before topk_run writes it
  topk_run<kLThreads, 32, kOneSeg>(K, max_cand, pos, mode, ratio, pool_len, cand_off, cand_idx, scores, stride,
                                   topk_idx, split, L);
}

}  // namespace

// Batches of at least this many queries take the survivor form for lists of
// one register segment, and the 512-thread shape for lists past one register
// segment or with Reindex lists.
constexpr int32_t kManyQueries = 512;
// Smaller batches with lists past one 1,024 x 16 segment split them over
// workgroups (kSegment) when given the buffers; the largest batches have
// workgroups enough without.
constexpr int32_t kSplitSeg = 1024 * 16;

static void launch_forms(int32_t K, int32_t B, const csa2_batch& bt, const float* scores, int64_t stride,
                         int32_t* topk_idx, hipStream_t s) {
  const TopkSplit none{0, nullptr, nullptr, nullptr, nullptr};
#define CSA2_TOPK_ARGS                                                                                    \
  K, bt.max_candidates, bt.pos, bt.mode, bt.compress_ratio, bt.pool_len, bt.cand_off, bt.cand_idx, scores, \
      stride, topk_idx, none
  // lists of at most one 512 x 32 segment and no Reindex lists: in a batch
  // of many queries the survivor form (several workgroups share each CU and
  // hide each other's barrier and LDS waits), otherwise the register-segment
  // form (one workgroup alone on a CU: its shorter chain of passes has the
  // lower latency; 11 against 15 us for 64 or 256 queries of 16,384)
  if (bt.max_candidates <= kLMax && bt.cand_off == nullptr && K <= kLThreads && B >= kManyQueries)
    hipLaunchKernelGGL(topk_lean_kernel, dim3(B), dim3(kLThreads), 0, s, CSA2_TOPK_ARGS);
  else if (bt.max_candidates <= 512 * 32 && bt.cand_off == nullptr)
    hipLaunchKernelGGL((topk_kernel<512, 32, kOneSeg>), dim3(B), dim3(512), 0, s, CSA2_TOPK_ARGS);
  else if (B >= kManyQueries)
    hipLaunchKernelGGL((topk_kernel<512, 32, kGeneral>), dim3(B), dim3(512), 0, s, CSA2_TOPK_ARGS);
  else
    hipLaunchKernelGGL((topk_kernel<1024, 16, kGeneral>), dim3(B), dim3(1024), 0, s, CSA2_TOPK_ARGS);
#undef CSA2_TOPK_ARGS
}

hipError_t launch_topk_k(int32_t K, int32_t B, const csa2_batch& bt, const float* scores, int64_t stride,
                         int32_t* topk_idx, hipStream_t s) {
  if (B == 0) return hipSuccess;
  launch_forms(K, B, bt, scores, stride, topk_idx, s);
  return hipGetLastError();
}

static int32_t split_segments(int32_t B, int32_t max_cand) {
  if (B <= 0 || B >= kManyQueries || max_cand <= kSplitSeg) return 0;
  return (max_cand + kSplitSeg - 1) / kSplitSeg;
}

size_t topk_split_bytes(int32_t B, int32_t max_cand) {
  const int32_t S = split_segments(B, max_cand);
  if (S == 0) return 0;
  const size_t a = 256;
  auto up = [&](size_t x) { return (x + a - 1) / a * a; };
  const size_t per = (size_t)B * S * kMaxTopK;
  return up(per * 4) + up(per * 4) + up((size_t)B * 4) + up(((size_t)B + 1) * 8);
}

hipError_t launch_topk(const csa2_dims& d, int32_t B, const csa2_batch& bt, const float* scores,
                       int64_t stride, int32_t* topk_idx, void* split_ws, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const int32_t K = d.index_topk;
  const int32_t S = split_segments(B, bt.max_candidates);
  if (split_ws == nullptr || S == 0 || K > kBins) {
    launch_forms(K, B, bt, scores, stride, topk_idx, s);
    return hipGetLastError();
  }
  const size_t a = 256;
  auto up = [&](size_t x) { return (x + a - 1) / a * a; };
  const size_t per = (size_t)B * S * kMaxTopK;
  uint8_t* p = static_cast<uint8_t*>(split_ws);
  TopkSplit sp;
  sp.nseg = S;
  sp.rows = reinterpret_cast<int32_t*>(p);
  sp.scores = reinterpret_cast<float*>(p + up(per * 4));
  sp.mode2 = reinterpret_cast<int32_t*>(p + 2 * up(per * 4));
  sp.off2 = reinterpret_cast<int64_t*>(p + 2 * up(per * 4) + up((size_t)B * 4));
  // each segment's top-K, then the top-K of those
  hipLaunchKernelGGL((topk_kernel<1024, 16, kSegment>), dim3(B, S), dim3(1024), 0, s, K, bt.max_candidates, bt.pos,
                     bt.mode, bt.compress_ratio, bt.pool_len, bt.cand_off, bt.cand_idx, scores, stride, topk_idx, sp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  csa2_batch b2 = bt;
  b2.mode = sp.mode2;
  b2.cand_off = sp.off2;
  b2.cand_idx = sp.rows;
  b2.max_candidates = S * K;
  // the merge's lists are short (S x K): a workgroup of 512 threads holding
  // four or eight keys each takes a query's list in one register segment,
  // at a fraction of the 1,024 x 16 form's latency
  const TopkSplit none{0, nullptr, nullptr, nullptr, nullptr};
#define CSA2_MERGE_ARGS                                                                                   \
  K, b2.max_candidates, b2.pos, b2.mode, b2.compress_ratio, b2.pool_len, b2.cand_off, b2.cand_idx, sp.scores, \
      (int64_t)S * K, topk_idx, none
  if (S * K <= 512 * 4)
    hipLaunchKernelGGL((topk_kernel<512, 4, kGeneral>), dim3(B), dim3(512), 0, s, CSA2_MERGE_ARGS);
  else if (S * K <= 512 * 8)
    hipLaunchKernelGGL((topk_kernel<512, 8, kGeneral>), dim3(B), dim3(512), 0, s, CSA2_MERGE_ARGS);
  else
    launch_forms(K, B, b2, sp.scores, (int64_t)S * K, topk_idx, s);
#undef CSA2_MERGE_ARGS
  return hipGetLastError();
}

}  // namespace csa2

