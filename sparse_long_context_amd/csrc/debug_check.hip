// Device-side precondition check of the entry points (CSA2_DEBUG_CHECK=1 in
// the environment).  Release calls trust the device arrays (positions,
// lengths, lists, selections, scale bytes) and only clamp their reads to the
// rows the descriptors describe; with the check on, a call first runs one
// kernel over those arrays that ORs a bit per violated precondition into an
// error word, reads the word back (the one synchronizing path of the
// library) and returns CSA2_ERR_PRECONDITION, launching nothing else, when a
// bit is set.  csa2_last_precondition() gives the word.
//
// A check reads only what the call itself would read: descriptors, lists and
// selections, the scale bytes of the KV rows a query can attend (its window
// rows; its pool rows up to its reachable count for Full / Reindex queries,
// its selected rows for Reuse), and, when the call scores, its index query,
// weights and the keys it scans.  A query whose descriptors are already wrong
// has none of its rows read.
#include <stdlib.h>

#include <mutex>

#include "csa2_internal.h"

namespace csa2 {
namespace {

__device__ uint32_t g_check_word;

__global__ void clear_word_kernel() { g_check_word = 0u; }

struct CheckArgs {
  csa2_batch bt;
  int32_t B, W, K, kv_dtype, key_dtype, index_heads;
  int32_t parts;
  const int32_t* sel;  // topk_idx (read for the selections the call attends), or NULL
  const float *idx_q, *idx_w;
  const void* idx_k;
  const uint8_t *idx_k_scale, *win_scale, *comp_scale;
};

__device__ __forceinline__ void flag(uint32_t bit) { atomicOr(&g_check_word, bit); }

// bytes of a KV scale plane row, and whether a byte of it decodes to NaN
__device__ __forceinline__ int scale_row_bytes(int kv) { return kv == CSA2_KV_FP8_E4M3_UE8M0_32 ? 16 : 32; }
__device__ __forceinline__ bool bad_scale(int kv, uint8_t v) {
  return kv == CSA2_KV_FP8_E4M3_UE8M0_32 ? v == 0xFFu : (v & 0x7Fu) == 0x7Fu;  // UE8M0 NaN / E4M3 NaN
}

__global__ __launch_bounds__(256) void check_kernel(CheckArgs a) {
  __shared__ int ok_s;
  const int b = blockIdx.x, t = threadIdx.x;
  const csa2_batch& bt = a.bt;
  if (t == 0) {
    uint32_t bits = 0;
    const int md = bt.mode[b];
    if (md < CSA2_MODE_FULL || md > CSA2_MODE_WINDOW) bits |= CSA2_PRE_MODE;
    if (bt.pos[b] < 0 || bt.compress_ratio[b] < 0 || bt.pool_len[b] < 0 || bt.pool_row0[b] < 0 || bt.win_row0[b] < 0 ||
        bt.win_len[b] < 0 || bt.win_len[b] > a.W)
      bits |= CSA2_PRE_DESC;
    if (md == CSA2_MODE_REINDEX && bt.cand_off && (bt.cand_off[b] < 0 || bt.cand_off[b + 1] < bt.cand_off[b]))
      bits |= CSA2_PRE_DESC;
    if (bits) flag(bits);
    ok_s = bits == 0;
  }
  __syncthreads();
  if (!ok_s) return;
  const int md = bt.mode[b];
  const int64_t nv = n_valid_of(bt.pos[b], bt.compress_ratio[b], md, bt.pool_len[b]);
  const bool selects = md == CSA2_MODE_FULL || md == CSA2_MODE_REINDEX;
  const int64_t prow0 = bt.pool_row0[b];

  // Reindex lists: strictly ascending rows, then only -1 padding
  if ((a.parts & kCheckLists) && md == CSA2_MODE_REINDEX && bt.cand_off) {
    const int64_t o0 = bt.cand_off[b], n = bt.cand_off[b + 1] - o0;
    for (int64_t j = t; j < n; j += blockDim.x) {
      const int32_t v = bt.cand_idx[o0 + j];
      const int32_t p = j > 0 ? bt.cand_idx[o0 + j - 1] : -2;
      if (v < -1 || (v >= 0 && j > 0 && (p == -1 || v <= p))) flag(CSA2_PRE_LIST);
    }
  }
  // selections the call attends: in [-1, pool_len), and their scale bytes
  const bool reads_sel = (a.parts & kCheckSelections) && a.sel && md != CSA2_MODE_WINDOW &&
                         (md == CSA2_MODE_REUSE || !(a.parts & kCheckSelectsOwn));
  if (reads_sel) {
    for (int j = t; j < a.K; j += blockDim.x) {
      const int32_t v = a.sel[(int64_t)b * a.K + j];
      if (v < -1 || v >= bt.pool_len[b]) {
        flag(CSA2_PRE_SEL);
      } else if (v >= 0 && a.comp_scale && a.kv_dtype != CSA2_KV_BF16) {
        const int sb = scale_row_bytes(a.kv_dtype);
        const uint8_t* p = a.comp_scale + (prow0 + v) * sb;
        for (int x = 0; x < sb; ++x)
          if (bad_scale(a.kv_dtype, p[x])) flag(CSA2_PRE_KV_SCALE);
      }
    }
  }
  if ((a.parts & kCheckScales) && a.kv_dtype != CSA2_KV_BF16) {
    const int sb = scale_row_bytes(a.kv_dtype);
    if (a.win_scale) {  // window rows
      const int64_t n = (int64_t)bt.win_len[b] * sb;
      const uint8_t* p = a.win_scale + bt.win_row0[b] * sb;
      for (int64_t x = t; x < n; x += blockDim.x)
        if (bad_scale(a.kv_dtype, p[x])) flag(CSA2_PRE_KV_SCALE);
    }
    if (a.comp_scale && selects && (a.parts & kCheckSelectsOwn)) {  // rows the query may select
      const int64_t n = nv * sb;
      const uint8_t* p = a.comp_scale + prow0 * sb;
      for (int64_t x = t; x < n; x += blockDim.x)
        if (bad_scale(a.kv_dtype, p[x])) flag(CSA2_PRE_KV_SCALE);
    }
  }
  // index inputs of a scoring call: finite q / weights / fp32 keys, MXFP4 key
  // scales that are not NaN (keys over the reachable rows: a Reindex list
  // names only such rows as eligible)
  if ((a.parts & kCheckIndex) && selects) {
    const int hi = a.index_heads;
    for (int x = t; x < hi * kIndexDim; x += blockDim.x)
      if (!isfinite(a.idx_q[(int64_t)b * hi * kIndexDim + x])) flag(CSA2_PRE_INDEX);
    if (a.idx_w)
      for (int x = t; x < hi; x += blockDim.x)
        if (!isfinite(a.idx_w[(int64_t)b * hi + x])) flag(CSA2_PRE_INDEX);
    if (a.key_dtype == CSA2_IDXK_F32) {
      const float* k = static_cast<const float*>(a.idx_k) + prow0 * kIndexDim;
      for (int64_t x = t; x < nv * kIndexDim; x += blockDim.x)
        if (!isfinite(k[x])) flag(CSA2_PRE_INDEX);
    } else {
      const uint8_t* s = a.idx_k_scale + prow0 * (kIndexDim / 32);
      for (int64_t x = t; x < nv * (kIndexDim / 32); x += blockDim.x)
        if (s[x] == 0xFFu) flag(CSA2_PRE_INDEX);
    }
  }
}

std::mutex g_check_mutex;
thread_local uint32_t g_last_word = 0;

}  // namespace

bool debug_check_enabled() {
  const char* e = getenv("CSA2_DEBUG_CHECK");
  return e && e[0] == '1' && e[1] == '\0';
}

uint32_t last_precondition_word() { return g_last_word; }

csa2_status debug_check(const csa2_dims& d, int32_t B, const csa2_batch& bt, int parts, const int32_t* sel,
                        const float* idx_q, const float* idx_w, const void* idx_k, const uint8_t* idx_k_scale,
                        const uint8_t* win_scale, const uint8_t* comp_scale, hipStream_t s) {
  g_last_word = 0;
  if (B == 0) return CSA2_OK;
  CheckArgs a;
  a.bt = bt;
  a.B = B;
  a.W = d.window;
  a.K = d.index_topk;
  a.kv_dtype = d.kv_dtype;
  a.key_dtype = d.index_key_dtype;
  a.index_heads = d.index_heads;
  a.parts = parts;
  a.sel = sel;
  a.idx_q = idx_q;
  a.idx_w = idx_w;
  a.idx_k = idx_k;
  a.idx_k_scale = idx_k_scale;
  a.win_scale = win_scale;
  a.comp_scale = comp_scale;
  if ((parts & kCheckIndex) && (!idx_q || !idx_k || (d.index_key_dtype == CSA2_IDXK_MXFP4 && !idx_k_scale)))
    a.parts &= ~kCheckIndex;
  // one check at a time per process: the word is one per device
  std::lock_guard<std::mutex> lock(g_check_mutex);
  hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(1), 0, s);
  hipLaunchKernelGGL(check_kernel, dim3(B), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  uint32_t word = 0;
  if (e == hipSuccess) e = hipMemcpyFromSymbolAsync(&word, HIP_SYMBOL(g_check_word), sizeof(word), 0,
                                                    hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return set_hip_error(e);
  g_last_word = word;
  return word ? CSA2_ERR_PRECONDITION : CSA2_OK;
}

}  // namespace csa2
