// Internal declarations shared by the kernels and the C-ABI layer of libcsa2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa2.h"

namespace csa2 {

constexpr int kHeads = 64;      // query heads sharing one KV row
constexpr int kDim = 512;       // dims per head and per KV row
constexpr int kIndexDim = 128;  // indexer key / query width
constexpr int kMaxIndexHeads = 64;
constexpr int kMaxCompressDim = 1024;  // widest latent the compressor pools
constexpr int kMaxRopeDims = 128;      // widest rope part the de-rotation turns
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

// Eight E2M1 codes (a 32-bit word, element 0 in the low nibble) -> their exact
// fp32 values, with the gfx950 scaled conversion at scale 1.
__device__ __forceinline__ void fp4x8_to_f32x8(uint32_t w, float* out) {
  const auto a0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const auto a1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const auto a2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const auto a3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  out[0] = a0[0], out[1] = a0[1], out[2] = a1[0], out[3] = a1[1];
  out[4] = a2[0], out[5] = a2[1], out[6] = a3[0], out[7] = a3[1];
}

// Eight E2M1 codes times a power of two 2^k (the float `scale`), each the
// exact product: the conversion takes only the exponent of its scale
// operand, which for a power of two is the whole scale.  The caller keeps
// every product a finite normal float (-125 <= k <= 125: magnitudes 0.5 .. 6).
__device__ __forceinline__ void fp4x8_pow2_to_f32x8(uint32_t w, float scale, float* out) {
  const auto a0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 0);
  const auto a1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 1);
  const auto a2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 2);
  const auto a3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 3);
  out[0] = a0[0], out[1] = a0[1], out[2] = a1[0], out[3] = a1[1];
  out[4] = a2[0], out[5] = a2[1], out[6] = a3[0], out[7] = a3[1];
}

// Eight E2M1 codes times one E4M3 scale byte -> eight bf16 (a uint4), exact:
// each product has at most 6 significant bits.
__device__ __forceinline__ uint4 fp4x8_e4m3_to_bf16x8(uint32_t w, uint32_t scale_byte) {
  float v[8];
  fp4x8_to_f32x8(w, v);
  const float s = __builtin_amdgcn_cvt_f32_fp8((int)scale_byte, 0);
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const __bf16 lo = (__bf16)(v[2 * i] * s), hi = (__bf16)(v[2 * i + 1] * s);
    o[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Output de-rotation ("DeepSeek-V4.1-Flash on WASTE", What is new, 1. CSA2:
// the rope dims of the attention output turn back by the query's rotation):
// the pair (off + 2i, off + 2i + 1) of every head turns by -pos * inv_freq[i],
// (x, y) -> (x cos a + y sin a, -x sin a + y cos a).  The angle, its cosine
// and sine are fp64, rounded to fp32; the turn is fp32 with one fused
// multiply-add per output, like the rest of the output arithmetic.  The fused
// epilogues and the standalone pass share these helpers, so both give the
// same bits.
constexpr int kRopePairs = kMaxRopeDims / 2;  // row width of a call's rope table
struct RopeOut {
  const double* inv_freq;  // nullptr: no de-rotation
  const float2* table;     // [B][kRopePairs] (cos, sin) per query, filled by launch_rope_table
  int32_t off, dims;       // even offset and dims, off + dims <= 512
};
__device__ __forceinline__ void rope_angle(int64_t pos, double f, float& cs, float& sn) {
  const double a = (double)pos * f;
  cs = (float)cos(a);
  sn = (float)sin(a);
}
__device__ __forceinline__ void rope_turn(float& x, float& y, float cs, float sn) {
  const float u = x, v = y;
  x = __builtin_fmaf(u, cs, v * sn);
  y = __builtin_fmaf(-u, sn, v * cs);
}
// The turns of one head's four output dims d0 .. d0 + 3 (d0 a multiple of 4,
// the offset even, so each pair lies inside): which of the two pairs are rope
// pairs, and their cosines and sines from the query's table row.
struct Rope4 {
  float c0, s0, c1, s1;
  bool t0, t1;
};
__device__ __forceinline__ Rope4 rope4_at(int d0, const float2* row, const RopeOut& r) {
  Rope4 q{1.f, 0.f, 1.f, 0.f, false, false};
  q.t0 = d0 >= r.off && d0 < r.off + r.dims;
  q.t1 = d0 + 2 >= r.off && d0 + 2 < r.off + r.dims;
  if (q.t0) {
    const float2 v = row[(d0 - r.off) >> 1];
    q.c0 = v.x, q.s0 = v.y;
  }
  if (q.t1) {
    const float2 v = row[(d0 + 2 - r.off) >> 1];
    q.c1 = v.x, q.s1 = v.y;
  }
  return q;
}
__device__ __forceinline__ float4 rope4_apply(float4 o, const Rope4& q) {
  if (q.t0) rope_turn(o.x, o.y, q.c0, q.s0);
  if (q.t1) rope_turn(o.z, o.w, q.c1, q.s1);
  return o;
}

// ---- launchers (each returns the launch's hipError_t) ----------------------

// Decode-shaped scores: one workgroup per (query, tile of candidates).
// idx_k: f32 keys, or MXFP4 codes with their E8M0 scale plane (d.index_key_dtype).
hipError_t launch_index_scores(const csa2_dims& d, int32_t B, const csa2_batch& bt, const float* idx_q,
                               const float* idx_w, const void* idx_k, const uint8_t* idx_k_scale,
                               float* scores, int64_t stride, hipStream_t s);
// Prefill-shaped scores (one sequence): register-tiled queries x candidates.
hipError_t launch_index_scores_prefill(const csa2_dims& d, int32_t T, const int64_t* pos, int32_t mode,
                                       int32_t ratio, int32_t pool_len, const float* idx_q,
                                       const float* idx_w, const float* idx_k, float* scores,
                                       int64_t stride, hipStream_t s);
// split_ws (topk_split_bytes, or NULL): lets a small batch with long lists
// spread each list over several workgroups
hipError_t launch_topk(const csa2_dims& d, int32_t B, const csa2_batch& bt, const float* scores,
                       int64_t stride, int32_t* topk_idx, void* split_ws, hipStream_t s);
size_t topk_split_bytes(int32_t B, int32_t max_cand);
// The same selection with an explicit K (any K >= 1).
hipError_t launch_topk_k(int32_t K, int32_t B, const csa2_batch& bt, const float* scores, int64_t stride,
                         int32_t* topk_idx, hipStream_t s);
// Hierarchical candidate pool of FULL queries (workspace: candidate_pool_ws_bytes).
size_t candidate_pool_ws_bytes(int32_t B, int32_t max_cand, int32_t block_size, int32_t top_blocks);
hipError_t launch_candidate_pool(int32_t B, const csa2_batch& bt, const float* scores, int64_t stride,
                                 int32_t block_size, int32_t top_blocks, int64_t* cand_off, int32_t* cand_idx,
                                 void* ws, hipStream_t s);
// n_split > 1 needs `partial` (see attend_partial_floats).
hipError_t launch_attend(const csa2_dims& d, int32_t B, const csa2_batch& bt, const void* q,
                         const void* win_kv, const uint8_t* win_scale, const void* comp_kv,
                         const uint8_t* comp_scale, const int32_t* topk_idx, const float* sink,
                         float* out, float* lse, int n_split, float* partial, const RopeOut& rope, hipStream_t s);
size_t attend_partial_floats(int32_t B, int n_split);
// Decode-shaped batches of fp8 / FP4 rows: four workgroups per query (16 heads
// each), no workspace; bf16 rows are refused (they take the all-heads kernel).
hipError_t launch_attend_hg(const csa2_dims& d, int32_t B, const csa2_batch& bt, const void* q,
                            const void* win_kv, const uint8_t* win_scale, const void* comp_kv,
                            const uint8_t* comp_scale, const int32_t* topk_idx, const float* sink, float* out,
                            float* lse, const RopeOut& rope, hipStream_t s);
// a query's entries go to at most this many (query, split) work items
constexpr int kMaxSplit = 4;
int attend_split_for(int32_t B);
// bf16 KV: resident workgroups of twelve waves (one per CU) taking (query,
// entry split) items in turn, rows gathered into LDS by DMA; n_split > 1
// needs `partial` (attend_partial_floats).
hipError_t launch_attend_mq(const csa2_dims& d, int32_t B, const csa2_batch& bt, const void* q,
                            const void* win_kv, const void* comp_kv, const int32_t* topk_idx, const float* sink,
                            float* out, float* lse, int n_split, float* partial, const RopeOut& rope,
                            hipStream_t s);
// Log-sum-exp merge of split partials into out / lse.
hipError_t launch_attend_combine(int32_t B, int n_split, const float* part_o, const float* part_ml, const float* sink,
                                 float* out, float* lse, const RopeOut& rope, hipStream_t s);

// The cache writer's quantizers (one thread per scale block).
hipError_t launch_quantize_fp4_kv(int64_t n_rows, int32_t d, const float* src, uint8_t* codes, uint8_t* scales,
                                  hipStream_t s);
hipError_t launch_quantize_mxfp4(int64_t n_rows, int32_t d, const float* src, uint8_t* codes, uint8_t* scales,
                                 hipStream_t s);

// Compressor (one workgroup per group) and output de-rotation (one per query).
hipError_t launch_compress(int64_t n_groups, int32_t m, int32_t d, const float* c, const float* g, const float* w,
                           float eps, float* out, hipStream_t s);
hipError_t launch_compress_step(int32_t B, int32_t m, int32_t d, const int64_t* pos, const float* c_new,
                                const float* g_new, float* kv_state, float* score_state, const float* w, float eps,
                                float* out, int32_t* emit_idx, hipStream_t s);
hipError_t launch_derotate(int32_t B, const int64_t* pos, int32_t rope_off, int32_t rope_dims,
                           const double* inv_freq, float* out, hipStream_t s);
// The (cos, sin) rows of a call's queries into r.table (rope_table_bytes(B)),
// for the attention kernels' fused de-rotation.
size_t rope_table_bytes(int32_t B);
hipError_t launch_rope_table(int32_t B, const int64_t* pos, const RopeOut& r, hipStream_t s);

// ---- device-side precondition check (CSA2_DEBUG_CHECK=1) ------------------
// parts of a call the check covers
constexpr int kCheckLists = 1;        // Reindex lists
constexpr int kCheckSelections = 2;   // topk_idx rows the call attends
constexpr int kCheckSelectsOwn = 4;   // the call selects for Full / Reindex queries itself
constexpr int kCheckScales = 8;       // KV scale bytes of the rows a query can attend
constexpr int kCheckIndex = 16;       // index query, weights and keys of the scoring
bool debug_check_enabled();
// Runs the check on `s` and waits for it: CSA2_OK, CSA2_ERR_PRECONDITION (the
// word is kept for csa2_last_precondition) or CSA2_ERR_HIP.
csa2_status debug_check(const csa2_dims& d, int32_t B, const csa2_batch& bt, int parts, const int32_t* sel,
                        const float* idx_q, const float* idx_w, const void* idx_k, const uint8_t* idx_k_scale,
                        const uint8_t* win_scale, const uint8_t* comp_scale, hipStream_t s);
uint32_t last_precondition_word();
// compute units of the current device (cached per device; 256 when it cannot
// be queried, e.g. with no GPU, so workspace sizes stay defined)
int device_cu_count();

// CSA2_TRACE=1: per-stage checksum lines on stderr (each waits for its stage)
bool trace_enabled();
void trace_scores(const char* call, int32_t B, const csa2_batch& bt, const float* scores, int64_t stride,
                  hipStream_t s);
void trace_topk(const char* call, int32_t B, const csa2_batch& bt, int32_t K, const int32_t* topk, hipStream_t s);
void trace_attend(const char* call, int32_t B, const float* out, const float* lse, hipStream_t s);

// records a failed HIP call for csa2_last_hip_error and returns CSA2_ERR_HIP
csa2_status set_hip_error(hipError_t e);

// csa2_decode on a given workspace (the caller's, or the static scratch)
csa2_status decode_impl(const csa2_dims* dims, int32_t B, const csa2_batch* batch, const void* q, const float* idx_q,
                        const float* idx_w, const void* idx_k, const uint8_t* idx_k_scale, const void* win_kv,
                        const uint8_t* win_scale, const void* comp_kv, const uint8_t* comp_scale, int32_t* topk_idx,
                        const float* sink, float* out, float* lse, void* workspace, size_t workspace_bytes,
                        const csa2_out_rope* rope, hipStream_t stream);

// Per-query descriptors of a prefill chunk, written into workspace arrays.
hipError_t launch_prefill_meta(const csa2_prefill_desc& p, int32_t window, int64_t* pos, int32_t* mode,
                               int32_t* ratio, int64_t* win_row0, int32_t* win_len, int64_t* pool_row0,
                               int32_t* pool_len, hipStream_t s);

}  // namespace csa2
