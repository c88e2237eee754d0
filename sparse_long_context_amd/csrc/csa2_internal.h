// Internal declarations shared by the kernels and the C-ABI layer of libcsa2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa2.h"

namespace csa2 {

constexpr int kHeads = 64;      // query heads sharing one KV row
constexpr int kDim = 512;       // dims per head and per KV row
constexpr int kIndexDim = 128;  // indexer key / query width
constexpr int kMaxTopK = 512;
constexpr int kMaxWindow = 128;
constexpr int kMaxEntries = kMaxWindow + kMaxTopK;  // 640 rows attended per query at most
constexpr int kScaleBlock = 32;                     // fp8 values per UE8M0 scale

// Number of reachable compressed entries of a query: entry j covers tokens
// j*m .. j*m+m-1 and is reachable once its last token is <= pos.
__device__ __forceinline__ int64_t n_valid_of(int64_t pos, int32_t m, int32_t mode, int32_t pool_len) {
  if (m <= 0 || mode == CSA2_MODE_WINDOW || pos < 0) return 0;
  int64_t n = (pos + 1) / m;
  return n < pool_len ? n : (int64_t)pool_len;
}

// ---- launchers (each returns the launch's hipError_t) ----------------------

// Decode-shaped scores: one workgroup per (query, tile of candidates).
hipError_t launch_index_scores(const csa2_dims& d, int32_t B, const csa2_batch& bt, const float* idx_q,
                               const float* idx_w, const float* idx_k, float* scores, int64_t stride,
                               hipStream_t s);
// Prefill-shaped scores (one sequence): register-tiled queries x candidates.
hipError_t launch_index_scores_prefill(const csa2_dims& d, int32_t T, const int64_t* pos, int32_t mode,
                                       int32_t ratio, int32_t pool_len, const float* idx_q,
                                       const float* idx_w, const float* idx_k, float* scores,
                                       int64_t stride, hipStream_t s);
hipError_t launch_topk(const csa2_dims& d, int32_t B, const csa2_batch& bt, const float* scores,
                       int64_t stride, int32_t* topk_idx, hipStream_t s);
// n_split > 1 needs `partial` (see attend_partial_floats).
hipError_t launch_attend(const csa2_dims& d, int32_t B, const csa2_batch& bt, const void* q,
                         const void* win_kv, const uint8_t* win_scale, const void* comp_kv,
                         const uint8_t* comp_scale, const int32_t* topk_idx, const float* sink,
                         float* out, float* lse, int n_split, float* partial, hipStream_t s);
size_t attend_partial_floats(int32_t B, int n_split);
// Decode-shaped batches: four workgroups per query (16 heads each), no workspace.
hipError_t launch_attend_hg(const csa2_dims& d, int32_t B, const csa2_batch& bt, const void* q,
                            const void* win_kv, const uint8_t* win_scale, const void* comp_kv,
                            const uint8_t* comp_scale, const int32_t* topk_idx, const float* sink, float* out,
                            float* lse, hipStream_t s);
int attend_split_for(int32_t B);

// Per-query descriptors of a prefill chunk, written into workspace arrays.
hipError_t launch_prefill_meta(const csa2_prefill_desc& p, int32_t window, int64_t* pos, int32_t* mode,
                               int32_t* ratio, int64_t* win_row0, int32_t* win_len, int64_t* pool_row0,
                               int32_t* pool_len, hipStream_t s);

}  // namespace csa2
