// C-ABI entry points of libcsa2 (declared in include/csa2.h): host-side
// validation, workspace carving and kernel launches.  Nothing here allocates,
// synchronizes or keeps a pointer.
#include <math.h>
#include <string.h>

#include <atomic>

#include "csa2_internal.h"

using namespace csa2;

namespace {

thread_local int32_t g_last_hip = 0;

csa2_status hip_status(hipError_t e) { return e == hipSuccess ? CSA2_OK : csa2::set_hip_error(e); }

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

csa2_status check_dims(const csa2_dims* d) {
  if (!d) return CSA2_ERR_INVALID_ARG;
  if (d->kv_dtype != CSA2_KV_BF16 && d->kv_dtype != CSA2_KV_FP8_E4M3_UE8M0_32 &&
      d->kv_dtype != CSA2_KV_FP4_E2M1_E4M3_16)
    return CSA2_ERR_INVALID_ARG;
  if (d->index_key_dtype != CSA2_IDXK_F32 && d->index_key_dtype != CSA2_IDXK_MXFP4) return CSA2_ERR_INVALID_ARG;
  if (d->index_relu != 0 && d->index_relu != 1) return CSA2_ERR_INVALID_ARG;
  if (!isfinite(d->softmax_scale)) return CSA2_ERR_INVALID_ARG;
  if (d->window < 0 || d->index_topk < 1 || d->index_heads < 1) return CSA2_ERR_INVALID_ARG;
  if (d->n_heads != kHeads || d->head_dim != kDim || d->index_dim != kIndexDim) return CSA2_ERR_UNSUPPORTED;
  if (d->window > kMaxWindow || d->index_topk > kMaxTopK || d->index_heads > kMaxIndexHeads)
    return CSA2_ERR_UNSUPPORTED;
  return CSA2_OK;
}

// Index keys need their scale plane exactly when they are MXFP4.
bool index_keys_ok(const csa2_dims* d, const void* idx_k, const uint8_t* idx_k_scale) {
  return idx_k && (d->index_key_dtype != CSA2_IDXK_MXFP4 || idx_k_scale);
}

csa2_status check_batch(const csa2_batch* bt, int32_t B) {
  if (!bt || B < 0) return CSA2_ERR_INVALID_ARG;
  if (B == 0) return CSA2_OK;
  if (!bt->pos || !bt->mode || !bt->compress_ratio || !bt->win_row0 || !bt->win_len || !bt->pool_row0 ||
      !bt->pool_len)
    return CSA2_ERR_INVALID_ARG;
  if (bt->max_candidates < 0) return CSA2_ERR_INVALID_ARG;
  if ((bt->cand_off == nullptr) != (bt->cand_idx == nullptr)) return CSA2_ERR_INVALID_ARG;
  return CSA2_OK;
}

size_t score_stride_for(int32_t max_cand) { return align_up((size_t)max_cand * sizeof(float)) / sizeof(float); }

// With fp8 / FP4 KV, batches of up to this many queries attend with four
// head-group workgroups per query (every workgroup streams all of its query's
// rows, sharing them through the XCD's L2); larger ones, and bf16 KV at any
// batch size, with workgroups of all 64 heads, where each row crosses into
// one CU only once (64 bf16 queries: 25.5 against the head groups' 31 us).
constexpr int32_t kHeadGroupMaxBatch = 64;
bool use_head_groups(const csa2_dims& d, int32_t B) {
  return B <= kHeadGroupMaxBatch && d.kv_dtype != CSA2_KV_BF16;
}

// Entry splits of the attention when a workspace is given (1: none).  The
// bf16 all-heads kernel splits only batches below 64 queries: from there on
// the merge of the partials costs more than the CUs the splits bring in
// (64 queries: 26.5 us split four ways, 25.5 unsplit; 128 queries: 30.4
// split two ways, 26.9 unsplit).
constexpr int32_t kMqSplitBelow = 64;
int all_heads_splits(const csa2_dims& d, int32_t B) {
  if (d.kv_dtype == CSA2_KV_BF16 && B >= kMqSplitBelow) return 1;
  return attend_split_for(B);
}
// the same for the decode and attention entry points, which send small fp8 /
// FP4 batches to the head groups (never split)
int attend_splits(const csa2_dims& d, int32_t B) { return use_head_groups(d, B) ? 1 : all_heads_splits(d, B); }

// Scores, then the split partials of the attention when its kernel uses them,
// then the rope table of a fused output de-rotation, then the top-K's split
// buffers (small batches with long lists).
size_t decode_ws_bytes(int32_t B, int32_t max_cand, int n_split) {
  size_t s = align_up((size_t)B * score_stride_for(max_cand) * sizeof(float));
  s += align_up(attend_partial_floats(B, n_split) * sizeof(float));
  s += align_up(rope_table_bytes(B));
  s += align_up(topk_split_bytes(B, max_cand));
  return s;
}
// where the top-K's split buffers start in that layout
size_t decode_ws_topk_offset(int32_t B, int32_t max_cand, int n_split) {
  return align_up((size_t)B * score_stride_for(max_cand) * sizeof(float)) +
         align_up(attend_partial_floats(B, n_split) * sizeof(float)) + align_up(rope_table_bytes(B));
}

// Per-query prefill descriptors live at the front of the prefill workspace.
struct PrefillMeta {
  int64_t* pos;
  int32_t* mode;
  int32_t* ratio;
  int64_t* win_row0;
  int32_t* win_len;
  int64_t* pool_row0;
  int32_t* pool_len;
};
size_t prefill_meta_bytes(int32_t T) { return 3 * align_up((size_t)T * 8) + 4 * align_up((size_t)T * 4); }
PrefillMeta carve_meta(uint8_t* p, int32_t T) {
  PrefillMeta m;
  const size_t a8 = align_up((size_t)T * 8), a4 = align_up((size_t)T * 4);
  m.pos = (int64_t*)p, p += a8;
  m.win_row0 = (int64_t*)p, p += a8;
  m.pool_row0 = (int64_t*)p, p += a8;
  m.mode = (int32_t*)p, p += a4;
  m.ratio = (int32_t*)p, p += a4;
  m.win_len = (int32_t*)p, p += a4;
  m.pool_len = (int32_t*)p;
  return m;
}
int32_t prefill_max_cand(const csa2_prefill_desc* p) {
  if (p->mode == CSA2_MODE_FULL) return p->pool_len;
  if (p->mode == CSA2_MODE_REINDEX) return p->max_candidates;
  return 0;
}

// The per-query batch view of a prefill chunk over its descriptor arrays.
csa2_batch prefill_batch(const csa2_prefill_desc* desc, const PrefillMeta& m, int32_t max_cand) {
  csa2_batch bt;
  bt.pos = m.pos;
  bt.mode = m.mode;
  bt.compress_ratio = m.ratio;
  bt.win_row0 = m.win_row0;
  bt.win_len = m.win_len;
  bt.pool_row0 = m.pool_row0;
  bt.pool_len = m.pool_len;
  bt.cand_off = desc->mode == CSA2_MODE_REINDEX ? desc->cand_off : nullptr;
  bt.cand_idx = desc->mode == CSA2_MODE_REINDEX ? desc->cand_idx : nullptr;
  bt.max_candidates = max_cand;
  return bt;
}

csa2_status check_prefill(const csa2_dims* d, const csa2_prefill_desc* p) {
  csa2_status st = check_dims(d);
  if (st != CSA2_OK) return st;
  if (!p || p->n_queries < 0 || p->pos0 < 0 || p->compress_ratio < 0 || p->pool_len < 0) return CSA2_ERR_INVALID_ARG;
  if (p->mode < CSA2_MODE_FULL || p->mode > CSA2_MODE_WINDOW) return CSA2_ERR_INVALID_ARG;
  if (p->win_pos0 < 0 || p->win_pos0 > p->pos0) return CSA2_ERR_INVALID_ARG;
  if (p->mode == CSA2_MODE_REINDEX && (!p->cand_off || !p->cand_idx || p->max_candidates < 0))
    return CSA2_ERR_INVALID_ARG;
  return CSA2_OK;
}

}  // namespace

namespace csa2 {
int device_cu_count() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cached[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

csa2_status set_hip_error(hipError_t e) {
  g_last_hip = (int32_t)e;
  return CSA2_ERR_HIP;
}
}  // namespace csa2

// ---- prefill descriptors ----------------------------------------------------
namespace csa2 {
namespace {
__global__ void prefill_meta_kernel(csa2_prefill_desc p, int32_t W, PrefillMeta m) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= p.n_queries) return;
  const int64_t pos = p.pos0 + t;
  int64_t lo = pos - W + 1;
  if (lo < p.win_pos0) lo = p.win_pos0;
  m.pos[t] = pos;
  m.mode[t] = p.mode;
  m.ratio[t] = p.compress_ratio;
  m.win_row0[t] = lo - p.win_pos0;
  m.win_len[t] = W > 0 ? (int32_t)(pos - lo + 1) : 0;
  m.pool_row0[t] = 0;
  m.pool_len[t] = p.pool_len;
}
}  // namespace
}  // namespace csa2

namespace {
// Scores of a prefill chunk: FULL chunks with one fp32-key index head score
// every query against the shared keys as one matrix product (whose tiles
// address 128 rows of scores with 32-bit byte offsets); any other form runs
// the decode-shaped kernels over the chunk's per-query view.
constexpr int64_t kPrefillScoreMaxStride = ((int64_t)1 << 23) - 64;
csa2_status prefill_scores(const csa2_dims* dims, const csa2_prefill_desc* desc, const csa2_batch& bt,
                           const PrefillMeta& m, const float* idx_q, const float* idx_w, const void* idx_k,
                           const uint8_t* idx_k_scale, float* scores, int64_t stride, hipStream_t stream) {
  const int32_t T = desc->n_queries;
  if (desc->mode == CSA2_MODE_FULL && dims->index_heads == 1 && dims->index_key_dtype == CSA2_IDXK_F32 &&
      stride <= kPrefillScoreMaxStride)
    return hip_status(launch_index_scores_prefill(*dims, T, m.pos, desc->mode, desc->compress_ratio, desc->pool_len,
                                                  idx_q, idx_w, static_cast<const float*>(idx_k), scores, stride,
                                                  stream));
  return hip_status(launch_index_scores(*dims, T, bt, idx_q, idx_w, idx_k, idx_k_scale, scores, stride, stream));
}
}  // namespace

extern "C" {

int csa2_abi_version(void) { return CSA2_ABI_VERSION; }

const char* csa2_status_str(csa2_status s) {
  switch (s) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_INVALID_ARG: return "invalid argument";
    case CSA2_ERR_UNSUPPORTED: return "unsupported geometry";
    case CSA2_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA2_ERR_HIP: return "HIP launch failed";
    case CSA2_ERR_PRECONDITION: return "device-side precondition failed (see csa2_last_precondition)";
  }
  return "unknown status";
}

int32_t csa2_last_hip_error(void) { return g_last_hip; }

uint32_t csa2_last_precondition(void) { return last_precondition_word(); }

csa2_status csa2_workspace_size(const csa2_dims* dims, int32_t B, int32_t max_candidates, size_t* bytes) {
  csa2_status st = check_dims(dims);
  if (st != CSA2_OK) return st;
  if (!bytes || B < 0 || max_candidates < 0) return CSA2_ERR_INVALID_ARG;
  *bytes = decode_ws_bytes(B, max_candidates, attend_splits(*dims, B));
  return CSA2_OK;
}

csa2_status csa2_index_scores(const csa2_dims* dims, int32_t B, const csa2_batch* batch, const float* idx_q,
                              const float* idx_w, const void* idx_k, const uint8_t* idx_k_scale, float* scores,
                              int64_t score_stride, hipStream_t stream) {
  csa2_status st = check_dims(dims);
  if (st == CSA2_OK) st = check_batch(batch, B);
  if (st != CSA2_OK) return st;
  if (B == 0 || batch->max_candidates == 0) return CSA2_OK;
  if (!idx_q || !index_keys_ok(dims, idx_k, idx_k_scale) || !scores || score_stride < batch->max_candidates)
    return CSA2_ERR_INVALID_ARG;
  if (debug_check_enabled() && (st = debug_check(*dims, B, *batch, kCheckLists | kCheckIndex, nullptr, idx_q, idx_w,
                                                 idx_k, idx_k_scale, nullptr, nullptr, stream)) != CSA2_OK)
    return st;
  return hip_status(
      launch_index_scores(*dims, B, *batch, idx_q, idx_w, idx_k, idx_k_scale, scores, score_stride, stream));
}

csa2_status csa2_topk(const csa2_dims* dims, int32_t B, const csa2_batch* batch, const float* scores,
                      int64_t score_stride, int32_t* topk_idx, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  csa2_status st = check_dims(dims);
  if (st == CSA2_OK) st = check_batch(batch, B);
  if (st != CSA2_OK) return st;
  if (B == 0) return CSA2_OK;
  if (!topk_idx || (batch->max_candidates > 0 && !scores) || score_stride < batch->max_candidates)
    return CSA2_ERR_INVALID_ARG;
  // the split buffers sit at the front of a workspace that is given
  if ((workspace == nullptr) != (workspace_bytes == 0)) return CSA2_ERR_INVALID_ARG;
  if (workspace && workspace_bytes < topk_split_bytes(B, batch->max_candidates)) return CSA2_ERR_WORKSPACE;
  if (debug_check_enabled() && (st = debug_check(*dims, B, *batch, kCheckLists, nullptr, nullptr, nullptr, nullptr,
                                                 nullptr, nullptr, nullptr, stream)) != CSA2_OK)
    return st;
  return hip_status(launch_topk(*dims, B, *batch, scores, score_stride, topk_idx, workspace, stream));
}

// Batches past the head-group size: with bf16 KV the all-heads kernel whose
// rows reach LDS by DMA; with fp8 / FP4 rows the all-heads kernel that stages
// rows through registers (both split a query's entries over several
// workgroups when the batch has fewer queries than CUs and a workspace).
static csa2_status attend_common(const csa2_dims* dims, int32_t B, const csa2_batch* batch, const void* q,
                                 const void* win_kv, const uint8_t* win_scale, const void* comp_kv,
                                 const uint8_t* comp_scale, const int32_t* topk_idx, const float* sink,
                                 float* out, float* lse, float* partial, int n_split, const RopeOut& rope,
                                 hipStream_t stream) {
  if (dims->kv_dtype == CSA2_KV_BF16)
    return hip_status(launch_attend_mq(*dims, B, *batch, q, win_kv, comp_kv, topk_idx, sink, out, lse, n_split,
                                       partial, rope, stream));
  return hip_status(launch_attend(*dims, B, *batch, q, win_kv, win_scale, comp_kv, comp_scale, topk_idx, sink,
                                  out, lse, n_split, partial, rope, stream));
}

static csa2_status check_attend_ptrs(const csa2_dims* dims, const void* q, const void* win_kv,
                                     const uint8_t* win_scale, const void* comp_kv, const uint8_t* comp_scale,
                                     float* out) {
  if (!q || !out) return CSA2_ERR_INVALID_ARG;
  if (dims->kv_dtype != CSA2_KV_BF16 && ((win_kv && !win_scale) || (comp_kv && !comp_scale)))
    return CSA2_ERR_INVALID_ARG;
  return CSA2_OK;
}

// The fused de-rotation's descriptor (NULL or rope_dims == 0: none).  Pairs
// must not straddle the four-dim columns the kernels store, hence the even
// offset.
static csa2_status rope_arg(const csa2_out_rope* r, RopeOut* out) {
  *out = RopeOut{nullptr, nullptr, 0, 0};
  if (!r) return CSA2_OK;
  if (r->rope_offset < 0 || (r->rope_offset % 2) != 0 || r->rope_dims < 0 || (r->rope_dims % 2) != 0 ||
      r->rope_dims > kMaxRopeDims || r->rope_offset + r->rope_dims > kDim)
    return CSA2_ERR_INVALID_ARG;
  if (r->rope_dims == 0) return CSA2_OK;
  if (!r->inv_freq) return CSA2_ERR_INVALID_ARG;
  *out = RopeOut{r->inv_freq, nullptr, r->rope_offset, r->rope_dims};
  return CSA2_OK;
}

// A fused de-rotation's table: its rows go to `table` (rope_table_bytes(B) of
// the workspace), filled for the call's queries before the attention runs.
static csa2_status rope_prepare(RopeOut& rope, int32_t B, const int64_t* pos, void* table, hipStream_t stream) {
  if (!rope.inv_freq) return CSA2_OK;
  rope.table = static_cast<const float2*>(table);
  return hip_status(launch_rope_table(B, pos, rope, stream));
}

csa2_status csa2_attend(const csa2_dims* dims, int32_t B, const csa2_batch* batch, const void* q,
                        const void* win_kv, const uint8_t* win_scale, const void* comp_kv,
                        const uint8_t* comp_scale, const int32_t* topk_idx, const float* sink, float* out,
                        float* lse, void* workspace, size_t workspace_bytes, const csa2_out_rope* rope_desc,
                        hipStream_t stream) {
  RopeOut rope;
  csa2_status st = check_dims(dims);
  if (st == CSA2_OK) st = check_batch(batch, B);
  if (st == CSA2_OK && B > 0) st = check_attend_ptrs(dims, q, win_kv, win_scale, comp_kv, comp_scale, out);
  if (st == CSA2_OK) st = rope_arg(rope_desc, &rope);
  if (st != CSA2_OK) return st;
  if (B == 0) return CSA2_OK;
  if (debug_check_enabled() &&
      (st = debug_check(*dims, B, *batch, kCheckSelections | kCheckScales, topk_idx, nullptr, nullptr, nullptr,
                        nullptr, win_scale, comp_scale, stream)) != CSA2_OK)
    return st;
  // workspace: the split partials (when the kernel splits), then the rope
  // table (when the output is de-rotated); none at all runs every query
  // unsplit, without de-rotation
  const bool no_ws = workspace == nullptr && workspace_bytes == 0;
  if (no_ws && rope.inv_freq) return CSA2_ERR_WORKSPACE;
  const int n_split = no_ws ? 1 : attend_splits(*dims, B);
  const size_t part_bytes = align_up(attend_partial_floats(B, n_split) * sizeof(float));
  const size_t need = part_bytes + (rope.inv_freq ? align_up(rope_table_bytes(B)) : 0);
  if (need > 0 && (!workspace || workspace_bytes < need)) return CSA2_ERR_WORKSPACE;
  if ((st = rope_prepare(rope, B, batch->pos, static_cast<uint8_t*>(workspace) + part_bytes, stream)) != CSA2_OK)
    return st;
  if (use_head_groups(*dims, B))
    return hip_status(launch_attend_hg(*dims, B, *batch, q, win_kv, win_scale, comp_kv, comp_scale, topk_idx, sink,
                                       out, lse, rope, stream));
  float* partial = n_split > 1 ? static_cast<float*>(workspace) : nullptr;
  return attend_common(dims, B, batch, q, win_kv, win_scale, comp_kv, comp_scale, topk_idx, sink, out, lse, partial,
                       n_split, rope, stream);
}

csa2_status csa2_decode(const csa2_dims* dims, int32_t B, const csa2_batch* batch, const void* q,
                        const float* idx_q, const float* idx_w, const void* idx_k, const uint8_t* idx_k_scale,
                        const void* win_kv,
                        const uint8_t* win_scale, const void* comp_kv, const uint8_t* comp_scale,
                        int32_t* topk_idx, const float* sink, float* out, float* lse, void* workspace,
                        size_t workspace_bytes, const csa2_out_rope* rope, hipStream_t stream) {
  return csa2::decode_impl(dims, B, batch, q, idx_q, idx_w, idx_k, idx_k_scale, win_kv, win_scale, comp_kv,
                           comp_scale, topk_idx, sink, out, lse, workspace, workspace_bytes, rope, stream);
}
}  // extern "C"

// The decode step on a given workspace; csa2_decode hands in the caller's,
// csa2_decode_static the library's static scratch.
csa2_status csa2::decode_impl(const csa2_dims* dims, int32_t B, const csa2_batch* batch, const void* q,
                              const float* idx_q, const float* idx_w, const void* idx_k, const uint8_t* idx_k_scale,
                              const void* win_kv, const uint8_t* win_scale, const void* comp_kv,
                              const uint8_t* comp_scale, int32_t* topk_idx, const float* sink, float* out,
                              float* lse, void* workspace, size_t workspace_bytes, const csa2_out_rope* rope_desc,
                              hipStream_t stream) {
  RopeOut rope;
  csa2_status st = check_dims(dims);
  if (st == CSA2_OK) st = check_batch(batch, B);
  if (st == CSA2_OK && B > 0) st = check_attend_ptrs(dims, q, win_kv, win_scale, comp_kv, comp_scale, out);
  if (st == CSA2_OK) st = rope_arg(rope_desc, &rope);
  if (st != CSA2_OK) return st;
  if (B == 0) return CSA2_OK;
  if (!topk_idx || (batch->max_candidates > 0 && (!idx_q || !index_keys_ok(dims, idx_k, idx_k_scale))))
    return CSA2_ERR_INVALID_ARG;
  const bool hg = use_head_groups(*dims, B);
  const size_t need = decode_ws_bytes(B, batch->max_candidates, attend_splits(*dims, B));
  if (need > 0 && (!workspace || workspace_bytes < need)) return CSA2_ERR_WORKSPACE;
  if (debug_check_enabled() &&
      (st = debug_check(*dims, B, *batch,
                        kCheckLists | kCheckSelections | kCheckSelectsOwn | kCheckScales |
                            (batch->max_candidates > 0 ? kCheckIndex : 0),
                        topk_idx, idx_q, idx_w, idx_k, idx_k_scale, win_scale, comp_scale, stream)) != CSA2_OK)
    return st;
  const int64_t stride = (int64_t)score_stride_for(batch->max_candidates);
  float* scores = static_cast<float*>(workspace);
  const int sp = attend_splits(*dims, B);
  uint8_t* after_scores = static_cast<uint8_t*>(workspace) + align_up((size_t)B * stride * sizeof(float));
  float* partial = sp > 1 ? reinterpret_cast<float*>(after_scores) : nullptr;
  if ((st = rope_prepare(rope, B, batch->pos, after_scores + align_up(attend_partial_floats(B, sp) * sizeof(float)),
                         stream)) != CSA2_OK)
    return st;

  // scores only when some candidate can exist; the top-K always runs, so
  // every FULL / REINDEX row of topk_idx is written (all -1 when nothing is
  // scored)
  const bool trace = trace_enabled();
  if (batch->max_candidates > 0 &&
      (st = hip_status(launch_index_scores(*dims, B, *batch, idx_q, idx_w, idx_k, idx_k_scale, scores, stride,
                                           stream))) != CSA2_OK)
    return st;
  if (trace) trace_scores("decode", B, *batch, scores, batch->max_candidates > 0 ? stride : 0, stream);
  void* split_ws = static_cast<uint8_t*>(workspace) + decode_ws_topk_offset(B, batch->max_candidates, sp);
  if ((st = hip_status(launch_topk(*dims, B, *batch, scores, stride, topk_idx, split_ws, stream))) != CSA2_OK)
    return st;
  if (trace) trace_topk("decode", B, *batch, dims->index_topk, topk_idx, stream);
  if (hg)
    st = hip_status(launch_attend_hg(*dims, B, *batch, q, win_kv, win_scale, comp_kv, comp_scale, topk_idx, sink,
                                     out, lse, rope, stream));
  else
    st = attend_common(dims, B, batch, q, win_kv, win_scale, comp_kv, comp_scale, topk_idx, sink, out, lse, partial,
                       sp, rope, stream);
  if (st == CSA2_OK && trace) trace_attend("decode", B, out, lse, stream);
  return st;
}

extern "C" {

csa2_status csa2_prefill_workspace_size(const csa2_dims* dims, const csa2_prefill_desc* desc, size_t* bytes) {
  csa2_status st = check_prefill(dims, desc);
  if (st != CSA2_OK) return st;
  if (!bytes) return CSA2_ERR_INVALID_ARG;
  const int32_t T = desc->n_queries;
  *bytes = prefill_meta_bytes(T) + decode_ws_bytes(T, prefill_max_cand(desc), all_heads_splits(*dims, T));
  return CSA2_OK;
}

csa2_status csa2_prefill_index_scores(const csa2_dims* dims, const csa2_prefill_desc* desc, const float* idx_q,
                                      const float* idx_w, const void* idx_k, const uint8_t* idx_k_scale, float* scores,
                                      int64_t score_stride, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  csa2_status st = check_prefill(dims, desc);
  if (st != CSA2_OK) return st;
  const int32_t T = desc->n_queries;
  const int32_t max_cand = prefill_max_cand(desc);
  if (T == 0 || max_cand == 0) return CSA2_OK;
  if (!idx_q || !index_keys_ok(dims, idx_k, idx_k_scale) || !scores || score_stride < max_cand ||
      (score_stride % 4) != 0)
    return CSA2_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < prefill_meta_bytes(T)) return CSA2_ERR_WORKSPACE;
  PrefillMeta m = carve_meta(static_cast<uint8_t*>(workspace), T);
  hipLaunchKernelGGL(prefill_meta_kernel, dim3((T + 255) / 256), dim3(256), 0, stream, *desc, dims->window, m);
  if ((st = hip_status(hipGetLastError())) != CSA2_OK) return st;
  csa2_batch bt = prefill_batch(desc, m, max_cand);
  if (debug_check_enabled() && (st = debug_check(*dims, T, bt, kCheckLists | kCheckIndex, nullptr, idx_q, idx_w,
                                                 idx_k, idx_k_scale, nullptr, nullptr, stream)) != CSA2_OK)
    return st;
  return prefill_scores(dims, desc, bt, m, idx_q, idx_w, idx_k, idx_k_scale, scores, score_stride, stream);
}

csa2_status csa2_prefill(const csa2_dims* dims, const csa2_prefill_desc* desc, const void* q, const float* idx_q,
                         const float* idx_w, const void* idx_k, const uint8_t* idx_k_scale, const void* win_kv,
                         const uint8_t* win_scale,
                         const void* comp_kv, const uint8_t* comp_scale, int32_t* topk_idx, const float* sink,
                         float* out, float* lse, void* workspace, size_t workspace_bytes,
                         const csa2_out_rope* rope_desc, hipStream_t stream) {
  RopeOut rope;
  csa2_status st = check_prefill(dims, desc);
  if (st == CSA2_OK) st = rope_arg(rope_desc, &rope);
  if (st != CSA2_OK) return st;
  const int32_t T = desc->n_queries;
  if (T == 0) return CSA2_OK;
  if ((st = check_attend_ptrs(dims, q, win_kv, win_scale, comp_kv, comp_scale, out)) != CSA2_OK) return st;
  const int32_t max_cand = prefill_max_cand(desc);
  const bool selects = desc->mode == CSA2_MODE_FULL || desc->mode == CSA2_MODE_REINDEX;
  if (desc->mode != CSA2_MODE_WINDOW && !topk_idx) return CSA2_ERR_INVALID_ARG;
  if (selects && max_cand > 0 && (!idx_q || !index_keys_ok(dims, idx_k, idx_k_scale))) return CSA2_ERR_INVALID_ARG;
  size_t need = prefill_meta_bytes(T) + decode_ws_bytes(T, max_cand, all_heads_splits(*dims, T));
  if (!workspace || workspace_bytes < need) return CSA2_ERR_WORKSPACE;

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  PrefillMeta m = carve_meta(ws, T);
  ws += prefill_meta_bytes(T);
  const int64_t stride = (int64_t)score_stride_for(max_cand);
  float* scores = reinterpret_cast<float*>(ws);
  ws += align_up((size_t)T * stride * sizeof(float));
  const int sp = all_heads_splits(*dims, T);
  float* partial = sp > 1 ? reinterpret_cast<float*>(ws) : nullptr;
  ws += align_up(attend_partial_floats(T, sp) * sizeof(float));

  hipLaunchKernelGGL(prefill_meta_kernel, dim3((T + 255) / 256), dim3(256), 0, stream, *desc, dims->window, m);
  if ((st = hip_status(hipGetLastError())) != CSA2_OK) return st;
  if ((st = rope_prepare(rope, T, m.pos, ws, stream)) != CSA2_OK) return st;
  csa2_batch bt = prefill_batch(desc, m, max_cand);
  if (debug_check_enabled() &&
      (st = debug_check(*dims, T, bt,
                        kCheckLists | kCheckSelections | kCheckSelectsOwn | kCheckScales |
                            (selects && max_cand > 0 ? kCheckIndex : 0),
                        desc->mode == CSA2_MODE_WINDOW ? nullptr : topk_idx, idx_q, idx_w, idx_k, idx_k_scale,
                        win_scale, comp_scale, stream)) != CSA2_OK)
    return st;

  const bool trace = trace_enabled();
  if (selects) {
    if (max_cand > 0 &&
        (st = prefill_scores(dims, desc, bt, m, idx_q, idx_w, idx_k, idx_k_scale, scores, stride, stream)) != CSA2_OK)
      return st;
    if (trace) trace_scores("prefill", T, bt, scores, max_cand > 0 ? stride : 0, stream);
    // always: with nothing scored every row becomes -1
    void* split_ws = static_cast<uint8_t*>(workspace) + prefill_meta_bytes(T) + decode_ws_topk_offset(T, max_cand, sp);
    if ((st = hip_status(launch_topk(*dims, T, bt, scores, stride, topk_idx, split_ws, stream))) != CSA2_OK) return st;
    if (trace) trace_topk("prefill", T, bt, dims->index_topk, topk_idx, stream);
  }
  st = attend_common(dims, T, &bt, q, win_kv, win_scale, comp_kv, comp_scale,
                     desc->mode == CSA2_MODE_WINDOW ? nullptr : topk_idx, sink, out, lse, partial, sp, rope, stream);
  if (st == CSA2_OK && trace) trace_attend("prefill", T, out, lse, stream);
  return st;
}

static csa2_status check_pool_args(int32_t B, int32_t max_cand, int32_t bs, int32_t top_blocks) {
  if (B < 0 || max_cand < 0 || bs < 1 || bs > 64 || top_blocks < 1 || top_blocks > 65536)
    return CSA2_ERR_INVALID_ARG;
  return CSA2_OK;
}

csa2_status csa2_candidate_pool_workspace_size(int32_t B, int32_t max_candidates, int32_t block_size,
                                               int32_t top_blocks, size_t* bytes) {
  csa2_status st = check_pool_args(B, max_candidates, block_size, top_blocks);
  if (st != CSA2_OK) return st;
  if (!bytes) return CSA2_ERR_INVALID_ARG;
  *bytes = candidate_pool_ws_bytes(B, max_candidates, block_size, top_blocks);
  return CSA2_OK;
}

csa2_status csa2_candidate_pool(int32_t B, const csa2_batch* batch, const float* scores, int64_t score_stride,
                                int32_t block_size, int32_t top_blocks, int64_t* cand_off, int32_t* cand_idx,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  csa2_status st = check_batch(batch, B);
  if (st != CSA2_OK) return st;
  if ((st = check_pool_args(B, batch ? batch->max_candidates : 0, block_size, top_blocks)) != CSA2_OK) return st;
  if (B == 0) return CSA2_OK;
  if (!cand_off || !cand_idx || (batch->max_candidates > 0 && !scores) || score_stride < batch->max_candidates)
    return CSA2_ERR_INVALID_ARG;
  const size_t need = candidate_pool_ws_bytes(B, batch->max_candidates, block_size, top_blocks);
  if (!workspace || workspace_bytes < need) return CSA2_ERR_WORKSPACE;
  if (debug_check_enabled()) {
    csa2_dims d{};
    d.window = kMaxWindow;
    d.index_topk = 1;
    if ((st = debug_check(d, B, *batch, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, stream)) !=
        CSA2_OK)
      return st;
  }
  return hip_status(launch_candidate_pool(B, *batch, scores, score_stride, block_size, top_blocks, cand_off, cand_idx,
                                          workspace, stream));
}

csa2_status csa2_compress(int64_t n_groups, int32_t m, int32_t d, const float* c, const float* g,
                          const float* norm_w, float eps, float* out, hipStream_t stream) {
  if (n_groups < 0 || m < 1 || d < 1 || d > kMaxCompressDim || !(eps >= 0.0f) || !isfinite(eps))
    return CSA2_ERR_INVALID_ARG;
  if (n_groups == 0) return CSA2_OK;
  if (!c || !norm_w || !out || (m > 1 && !g)) return CSA2_ERR_INVALID_ARG;
  return hip_status(launch_compress(n_groups, m, d, c, g, norm_w, eps, out, stream));
}

csa2_status csa2_compress_step(int32_t B, int32_t m, int32_t d, const int64_t* pos, const float* c_new,
                               const float* g_new, float* kv_state, float* score_state, const float* norm_w, float eps,
                               float* out, int32_t* emit_idx, hipStream_t stream) {
  if (B < 0 || m < 1 || d < 1 || d > kMaxCompressDim || !(eps >= 0.0f) || !isfinite(eps))
    return CSA2_ERR_INVALID_ARG;
  if (B == 0) return CSA2_OK;
  if (!pos || !c_new || !norm_w || !out || !emit_idx || (m > 1 && (!g_new || !kv_state || !score_state)))
    return CSA2_ERR_INVALID_ARG;
  return hip_status(
      launch_compress_step(B, m, d, pos, c_new, g_new, kv_state, score_state, norm_w, eps, out, emit_idx, stream));
}

csa2_status csa2_derotate(const csa2_dims* dims, int32_t B, const int64_t* pos, int32_t rope_offset,
                          int32_t rope_dims, const double* inv_freq, float* out, hipStream_t stream) {
  csa2_status st = check_dims(dims);
  if (st != CSA2_OK) return st;
  if (B < 0 || rope_offset < 0 || rope_dims < 0 || (rope_dims % 2) != 0 || rope_dims > kMaxRopeDims ||
      rope_offset + rope_dims > kDim)
    return CSA2_ERR_INVALID_ARG;
  if (B == 0 || rope_dims == 0) return CSA2_OK;
  if (!pos || !inv_freq || !out) return CSA2_ERR_INVALID_ARG;
  return hip_status(launch_derotate(B, pos, rope_offset, rope_dims, inv_freq, out, stream));
}

csa2_status csa2_quantize_fp4_kv(int64_t n_rows, int32_t d, const float* src, uint8_t* codes, uint8_t* scales,
                                 hipStream_t stream) {
  if (n_rows < 0 || d <= 0 || (d % 16) != 0) return CSA2_ERR_INVALID_ARG;
  if (n_rows == 0) return CSA2_OK;
  if (!src || !codes || !scales) return CSA2_ERR_INVALID_ARG;
  return hip_status(launch_quantize_fp4_kv(n_rows, d, src, codes, scales, stream));
}

csa2_status csa2_quantize_mxfp4(int64_t n_rows, int32_t d, const float* src, uint8_t* codes, uint8_t* scales,
                                hipStream_t stream) {
  if (n_rows < 0 || d <= 0 || (d % 32) != 0) return CSA2_ERR_INVALID_ARG;
  if (n_rows == 0) return CSA2_OK;
  if (!src || !codes || !scales) return CSA2_ERR_INVALID_ARG;
  return hip_status(launch_quantize_mxfp4(n_rows, d, src, codes, scales, stream));
}

}  // extern "C"
