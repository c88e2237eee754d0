/*
 * csa2.h -- C ABI of the CSA2 compressed-sparse-attention step on MI355X (gfx950).
 *
 * What the step computes (one query token):
 *   1. Reachability: compressed entry j stands for the m tokens j*m .. j*m+m-1
 *      and can be read once its last token is at or before the query position
 *      ("Reading Notes of DeepSeek-V4.1-Flash", section 3f C2 Step 1; PocketLLM
 *      "DeepSeek-V4.1-Flash", "The CSA2 attention layers": a partial group emits
 *      nothing).  n_valid = min(pool_len, floor((pos + 1) / m)); m = 0 -> 0.
 *   2. Index scores: sigma(j) = sum_h w_h * f(q^I_h . k^I_j), f = ReLU or identity
 *      (Reading Notes, 3f C2 Step 2, lightning-indexer form).
 *   3. Top-K: keep the K best candidates (same section), lowest index winning a
 *      tie; unused slots hold -1 (PocketLLM page, "Correctness and precision").
 *   4. Attention: the query's H heads attend in ONE softmax over the
 *      concatenation of its sliding window of raw KV rows and the selected
 *      compressed rows; each KV row is both key and value (one 512-wide KV per
 *      token shared by all heads: "DeepSeek-V4.1-Flash on WASTE", What is new,
 *      1. CSA2; Reading Notes, 3f C2 Step 3).  An optional per-head sink logit
 *      joins the denominator only (WASTE page, same section).  A query with no
 *      entry returns zeros (PocketLLM page, "The op layer": finite score floor).
 *   Modes (Reading Notes, 3f C2 Step 4): FULL scores every reachable entry;
 *   REINDEX scores a supplied candidate list (3f C3: a later layer searches
 *   only its pool); REUSE takes a supplied selection; WINDOW has no
 *   compressed branch (compress ratio 0).
 *
 * Numerics.  Index scores are fp32 with a fixed evaluation order, so selections
 * are reproducible bit for bit: per head acc = +0, acc = fmaf(q[i], k[i], acc)
 * for i = 0 .. D_I-1 in order; f applied; s = +0, s = fmaf(w_h, f_h, s) for
 * h = 0 .. H_I-1 in order (w_h = 1 when no weights are given); -0 becomes +0.
 * Attention multiplies bf16 operands on the matrix cores with fp32
 * accumulation and an fp32 online softmax; the probabilities are rounded to
 * bf16 for the second product.  FP8 KV (E4M3, one UE8M0 scale per 32 values)
 * and FP4 KV (E2M1, one E4M3 scale per 16 values: Reading Notes, 3f C4) are
 * widened to bf16 exactly before use; MXFP4 index keys (E2M1, one E8M0 scale
 * per 32: PocketLLM page, "The CSA2 attention layers") are widened to fp32
 * exactly before the fixed-order score.
 *
 * Conventions common to every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; nothing is
 *     retained after the call returns.  Base pointers are 16-byte aligned.
 *   - Calls only enqueue work on `stream` and never synchronize.
 *   - The library is stateless and allocates no device memory; scratch comes
 *     from a caller-provided workspace sized by the *_workspace_size calls.
 *   - Host-visible arguments are validated before anything is launched; on an
 *     error nothing is launched and no output is touched.  A failed launch
 *     returns CSA2_ERR_HIP and csa2_last_hip_error() gives its hipError_t.
 *   - Device-side values (positions, lengths, indices) are preconditions; every
 *     kernel clamps its reads to the rows the descriptors describe, so a bad
 *     index yields a wrong answer, never an access outside the described rows.
 *   - Supported geometry: n_heads 64, head_dim 512, index_dim 128,
 *     1 <= index_heads <= 64, 1 <= index_topk <= 512, 0 <= window <= 128.
 *     Others return CSA2_ERR_UNSUPPORTED.
 *
 * Layouts (row-major, rows contiguous):
 *   q        bf16  [B][64][512]
 *   idx_q    f32   [B][H_I][128];  idx_w f32 [B][H_I] or NULL (unit weights)
 *   idx_k    f32   [rows][128]     (same row numbering as comp_kv), or MXFP4:
 *            codes uint8 [rows][64] with idx_k_scale uint8 [rows][4]
 *            (E8M0, value = code * 2^(s-127), one scale per 32 values)
 *   win_kv / comp_kv: bf16 [rows][512], or fp8 codes uint8 [rows][512] with
 *            scales uint8 [rows][16] (UE8M0, value = code * 2^(s-127), s = 0 .. 254;
 *            255 is NaN and not allowed; decoded values below 2^-126 in magnitude
 *            may be flushed to zero in the bf16 / fp32 arithmetic), or FP4
 *            codes uint8 [rows][256] with scales uint8 [rows][32] (E4M3,
 *            value = code * scale, one scale per 16 values)
 *   FP4 codes: E2M1 (0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6), two per byte,
 *            element 2i in the low nibble.
 *   topk_idx int32 [B][K]: pool-relative row numbers, ascending, -1 padded
 *   out      f32   [B][64][512];   lse f32 [B][64] (natural log) or NULL
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_ABI_VERSION 4

typedef enum {
  CSA2_OK = 0,
  CSA2_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad enum, ... */
  CSA2_ERR_UNSUPPORTED = 2, /* geometry this build does not implement */
  CSA2_ERR_WORKSPACE = 3,   /* workspace missing or too small */
  CSA2_ERR_HIP = 4,         /* a kernel launch failed; see csa2_last_hip_error */
  CSA2_ERR_PRECONDITION = 5 /* CSA2_DEBUG_CHECK=1 only: a device-side precondition does not
                               hold; see csa2_last_precondition */
} csa2_status;

/* Bits of the device-side precondition word (csa2_last_precondition). */
#define CSA2_PRE_MODE 1u      /* a mode outside FULL .. WINDOW */
#define CSA2_PRE_DESC 2u      /* a negative position / ratio / row0 / length, win_len above the
                                 window, or decreasing cand_off */
#define CSA2_PRE_LIST 4u      /* a Reindex list that is not strictly ascending before its -1
                                 padding, or holds an entry below -1 */
#define CSA2_PRE_SEL 8u       /* an attended topk_idx entry outside [-1, pool_len) */
#define CSA2_PRE_KV_SCALE 16u /* an fp8 / FP4 scale byte that decodes to NaN in a row the query
                                 can attend */
#define CSA2_PRE_INDEX 32u    /* a non-finite index query, weight or fp32 key, or an MXFP4 key
                                 scale byte 255, in what the call scores */

typedef enum {
  CSA2_KV_BF16 = 0,
  CSA2_KV_FP8_E4M3_UE8M0_32 = 1, /* sliding-window format of the pages' model */
  CSA2_KV_FP4_E2M1_E4M3_16 = 2   /* main (compressed) KV format, Reading Notes 3f C4 */
} csa2_kv_dtype;

typedef enum {
  CSA2_IDXK_F32 = 0,  /* fp32 keys */
  CSA2_IDXK_MXFP4 = 1 /* E2M1 codes + E8M0 scale per 32 */
} csa2_index_key_dtype;

typedef enum {
  CSA2_MODE_FULL = 0,    /* score every reachable compressed entry, select top-K */
  CSA2_MODE_REINDEX = 1, /* score a supplied candidate list, select top-K */
  CSA2_MODE_REUSE = 2,   /* attend a supplied selection */
  CSA2_MODE_WINDOW = 3   /* window rows only */
} csa2_mode;

typedef struct csa2_dims {
  int32_t n_heads;     /* H, query heads (64) */
  int32_t head_dim;    /* D, dims per head and per KV row (512) */
  int32_t window;      /* W, window rows per query, at most (prefill: the window size) */
  int32_t index_topk;  /* K, selected compressed entries per query */
  int32_t index_dim;   /* D_I (128) */
  int32_t index_heads; /* H_I */
  int32_t index_relu;  /* 0: f = identity, 1: f = ReLU */
  int32_t kv_dtype;    /* csa2_kv_dtype, for both KV sources */
  float softmax_scale; /* multiplies q.k before the softmax (1 when folded into q) */
  int32_t index_key_dtype; /* csa2_index_key_dtype of idx_k */
} csa2_dims;

/* Per-query descriptors of a decode batch: DEVICE arrays of length B (cand_off: B+1). */
typedef struct csa2_batch {
  const int64_t *pos;            /* absolute position of the query token */
  const int32_t *mode;           /* csa2_mode */
  const int32_t *compress_ratio; /* m; 0 = no compressed branch */
  const int64_t *win_row0;       /* first window row of the query in win_kv */
  const int32_t *win_len;        /* its number of window rows, 0 .. W (order free) */
  const int64_t *pool_row0;      /* first row of the query's pool in comp_kv / idx_k */
  const int32_t *pool_len;       /* rows in that pool */
  const int64_t *cand_off;       /* REINDEX: list of query b is cand_idx[cand_off[b] .. cand_off[b+1]) */
  const int32_t *cand_idx;       /*   pool-relative rows, strictly ascending, optionally followed by -1
                                    padding (never eligible); NULL if no REINDEX query */
  int32_t max_candidates;        /* HOST value: candidates considered per FULL/REINDEX query are
                                    capped at this (use the largest pool_len / list length) */
} csa2_batch;

/* One prefill chunk: T consecutive queries of one sequence (host values). */
typedef struct csa2_prefill_desc {
  int64_t pos0;           /* position of the first query; query t sits at pos0 + t */
  int32_t n_queries;      /* T */
  int32_t mode;           /* csa2_mode, the same for the whole chunk */
  int32_t compress_ratio; /* m */
  int32_t pool_len;       /* rows of comp_kv / idx_k (the sequence's whole pool) */
  int64_t win_pos0;       /* win_kv row r holds position win_pos0 + r.  It is also the replay
                             start: a window never reaches before it (Reading Notes, 3f C5,
                             SWA bounded replay).  Query at p reads rows
                             [max(win_pos0, p - W + 1), p] - win_pos0.  Needs win_pos0 <= pos0. */
  const int64_t *cand_off; /* REINDEX (device, T+1) / NULL */
  const int32_t *cand_idx;
  int32_t max_candidates;  /* REINDEX: cap on list length per query (host); ignored otherwise */
} csa2_prefill_desc;

/* Output de-rotation fused into the attention's output writes ("DeepSeek-V4.1-
 * Flash on WASTE", What is new, 1. CSA2: the rope dims of the output turn back
 * by the query's own rotation).  Passed as `rope` to csa2_attend, csa2_decode,
 * csa2_decode_static and csa2_prefill (NULL: outputs left as attended): the
 * output of query b is written already turned exactly as csa2_derotate would
 * turn it with pos[b] (same bits), saving that pass's read and write of
 * `out`.  rope_offset and rope_dims even, rope_dims <= 128, rope_offset +
 * rope_dims <= 512; inv_freq: device f64 [rope_dims / 2]; rope_dims == 0
 * turns nothing.  Invalid fields: CSA2_ERR_INVALID_ARG.  The call's cosines
 * and sines go to a 512-byte row per query of its workspace (counted in
 * csa2_workspace_size and csa2_prefill_workspace_size), so csa2_attend needs
 * a workspace for it (none: CSA2_ERR_WORKSPACE). */
typedef struct csa2_out_rope {
  int32_t rope_offset;
  int32_t rope_dims;
  const double *inv_freq;
} csa2_out_rope;

int csa2_abi_version(void);
const char *csa2_status_str(csa2_status s);
/* hipError_t of the last CSA2_ERR_HIP returned on this thread (0 if none). */
int32_t csa2_last_hip_error(void);
/* Precondition word (CSA2_PRE_* bits) of the last call on this thread that
 * ran the device-side check: 0 when it passed or no call ran it.
 *
 * Device-side check.  Release calls trust device arrays: positions, lengths,
 * lists, selections and scale bytes are preconditions (see "Conventions").
 * With CSA2_DEBUG_CHECK=1 in the environment (read at every call), each of
 * csa2_index_scores, csa2_topk, csa2_attend, csa2_decode, csa2_prefill and
 * csa2_candidate_pool first runs one kernel over what the call will read, then
 * reads the word back and waits for it on `stream` (the only synchronizing
 * path of the library, so it cannot run under graph capture: CSA2_ERR_HIP
 * then).  If a bit is set the call returns CSA2_ERR_PRECONDITION and launches
 * nothing else (csa2_prefill has by then written only its workspace).  Checks
 * of concurrent calls in one process run one at a time. */
uint32_t csa2_last_precondition(void);

/* Trace.  With CSA2_TRACE=1 in the environment (read at every call),
 * csa2_decode, csa2_decode_static and csa2_prefill print one checksum line per
 * stage on stderr, in the format of the oracle's trace for the same results:
 *   csa2-trace <call> scores finite=<n> sum=<s>   (fp64 sum of the finite
 *       scores of the Full / Reindex queries, query by query in candidate
 *       order: equal to the oracle's, digit for digit)
 *   csa2-trace <call> topk rows=<r> chosen=<c> fnv1a=<h>   (the top-K rows
 *       written: entries >= 0, and the 64-bit FNV-1a hash of their int32
 *       values, little-endian, row by row)
 *   csa2-trace <call> attend out_sum=<s> out_abs=<a> lse_sum=<l> lse_ninf=<k>
 * Each line waits for its stage on `stream` and copies its output to the
 * host: a debugging aid that cannot run under graph capture. */

/* Workspace bytes csa2_decode needs for B queries with at most max_candidates
 * candidates each (scores, plus the partials of the attention's entry splits,
 * which it takes for bf16 batches below 64 queries and fp8 / FP4 batches of
 * 65 to 255, plus 512 bytes per query for a fused output de-rotation).  With
 * max_candidates = 0 it is the workspace csa2_attend can use to split entries
 * and to de-rotate. */
csa2_status csa2_workspace_size(const csa2_dims *dims, int32_t B, int32_t max_candidates,
                                size_t *bytes);

/* Steps 1-2 for every FULL / REINDEX query b of the batch (other queries are
 * skipped): scores[b * score_stride + j] for candidate j < n_cand(b), where
 * n_cand = min(n_valid, max_candidates) (FULL: candidate j is pool row j) or
 * min(list length, max_candidates) (REINDEX: candidate j is the j-th list row).
 * A listed row outside [0, n_valid) scores -inf.  Other slots are not written.
 * Requires score_stride >= max_candidates.  idx_k is f32 keys, or MXFP4 codes
 * with their scale plane idx_k_scale (dims->index_key_dtype; idx_k_scale is
 * ignored for f32 keys). */
csa2_status csa2_index_scores(const csa2_dims *dims, int32_t B, const csa2_batch *batch,
                              const float *idx_q, const float *idx_w, const void *idx_k,
                              const uint8_t *idx_k_scale, float *scores, int64_t score_stride,
                              hipStream_t stream);

/* Step 3 for every FULL / REINDEX query: from the scores of csa2_index_scores,
 * write the first min(K, eligible) candidates under (score descending, row
 * ascending) to topk_idx[b][*] in ascending row order, padded with -1.
 * Eligible: candidate row in [0, n_valid).  Scores must be finite or -inf; +0
 * and -0 tie.  Rows of REUSE / WINDOW queries are not written.
 * workspace: NULL (workspace_bytes 0), or at least
 * csa2_workspace_size(dims, B, batch->max_candidates) bytes, with which a
 * batch of under 512 queries whose lists exceed 16,384 candidates spreads
 * each list over several workgroups (each keeps its segment's K best, then
 * the K best of those are taken: the same result). */
csa2_status csa2_topk(const csa2_dims *dims, int32_t B, const csa2_batch *batch, const float *scores,
                      int64_t score_stride, int32_t *topk_idx, void *workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* Step 4 for every query: FULL / REINDEX / REUSE queries attend their window
 * rows plus the pool rows named in topk_idx[b] (-1 skipped; duplicates count
 * per occurrence; rows outside [0, pool_len) skipped); WINDOW queries attend
 * their window rows only (topk_idx may be NULL if every query is WINDOW).
 * win_kv may be NULL (no query then has window rows) and comp_kv may be NULL
 * (no query then has compressed rows); the scale planes of fp8 / FP4 KV are
 * required exactly when their KV source is given.
 * sink: f32 [64] or NULL.
 * With fp8 / FP4 KV, batches of B <= 64 queries run four workgroups of 16
 * heads per query and ignore the workspace.  Larger batches, and bf16 KV at
 * every B, run workgroups of all 64 heads; with a workspace of
 * csa2_workspace_size(dims, B, 0) bytes the entries of a query may be split
 * over several such workgroups and merged, with workspace == NULL and
 * workspace_bytes == 0 every query runs unsplit (and `rope` must be NULL). */
csa2_status csa2_attend(const csa2_dims *dims, int32_t B, const csa2_batch *batch, const void *q,
                        const void *win_kv, const uint8_t *win_scale, const void *comp_kv,
                        const uint8_t *comp_scale, const int32_t *topk_idx, const float *sink,
                        float *out, float *lse, void *workspace, size_t workspace_bytes,
                        const csa2_out_rope *rope, hipStream_t stream);

/* The whole step for a decode batch of independent queries with per-query
 * modes: scores + top-K for FULL / REINDEX queries (their topk_idx rows are
 * written), then attention for all (REUSE rows of topk_idx are read). */
csa2_status csa2_decode(const csa2_dims *dims, int32_t B, const csa2_batch *batch, const void *q,
                        const float *idx_q, const float *idx_w, const void *idx_k,
                        const uint8_t *idx_k_scale, const void *win_kv, const uint8_t *win_scale, const void *comp_kv,
                        const uint8_t *comp_scale, int32_t *topk_idx, const float *sink,
                        float *out, float *lse, void *workspace, size_t workspace_bytes,
                        const csa2_out_rope *rope, hipStream_t stream);

/* csa2_decode for callers that cannot allocate device memory (work captured
 * into a HIP graph, serving loops or harnesses that forbid allocation): the
 * same step with the same arguments and results, but no workspace argument.
 * Its scratch is a static device array of CSA2_STATIC_SCRATCH_BYTES held by
 * every GPU the library runs on until the process ends; the call allocates
 * and frees nothing.  It returns CSA2_ERR_WORKSPACE, launching nothing, when
 * csa2_workspace_size(dims, B, batch->max_candidates) exceeds that size (e.g.
 * 64 queries x 16,384 candidates need 4 MiB, 128 x 65,536 need 32 MiB).  Calls
 * that overlap on one GPU (other streams or threads) share the array and
 * race: serialize them. */
#define CSA2_STATIC_SCRATCH_BYTES (64u << 20)
csa2_status csa2_decode_static(const csa2_dims *dims, int32_t B, const csa2_batch *batch, const void *q,
                               const float *idx_q, const float *idx_w, const void *idx_k,
                               const uint8_t *idx_k_scale, const void *win_kv, const uint8_t *win_scale,
                               const void *comp_kv, const uint8_t *comp_scale, int32_t *topk_idx,
                               const float *sink, float *out, float *lse, const csa2_out_rope *rope,
                               hipStream_t stream);

/* Workspace bytes for csa2_prefill on this chunk. */
csa2_status csa2_prefill_workspace_size(const csa2_dims *dims, const csa2_prefill_desc *desc,
                                        size_t *bytes);

/* Steps 1-2 for a FULL / REINDEX prefill chunk: scores[t * score_stride + j]
 * for query t and its candidate j, exactly as csa2_index_scores defines them
 * for the query at pos0 + t (FULL: candidate j is pool row j, j < n_valid;
 * REINDEX: the j-th row of its list, unreachable rows -inf); other slots are
 * not written.  Requires score_stride >= the chunk's candidate cap (pool_len
 * for FULL, max_candidates for REINDEX) and a multiple of 4 (scores are
 * stored 16 bytes at a time; `scores` is 16-byte aligned like every base).  The workspace is that of
 * csa2_prefill (csa2_prefill_workspace_size).  Other modes: nothing to do. */
csa2_status csa2_prefill_index_scores(const csa2_dims *dims, const csa2_prefill_desc *desc, const float *idx_q,
                                      const float *idx_w, const void *idx_k, const uint8_t *idx_k_scale,
                                      float *scores, int64_t score_stride, void *workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* The whole step for one prefill chunk (T queries of one sequence sharing its
 * window rows, pool and index keys).  Per query t at p = pos0 + t: window rows
 * as in csa2_prefill_desc; reachability, scores and top-K as for decode; q,
 * idx_q, topk_idx, out and lse are indexed by t. */
csa2_status csa2_prefill(const csa2_dims *dims, const csa2_prefill_desc *desc, const void *q,
                         const float *idx_q, const float *idx_w, const void *idx_k,
                         const uint8_t *idx_k_scale, const void *win_kv, const uint8_t *win_scale, const void *comp_kv,
                         const uint8_t *comp_scale, int32_t *topk_idx, const float *sink,
                         float *out, float *lse, void *workspace, size_t workspace_bytes,
                         const csa2_out_rope *rope, hipStream_t stream);

/* Hierarchical candidate pool (Reading Notes, 3f C3; PocketLLM page, "The
 * CSA2 attention layers"): from the scores csa2_index_scores wrote for the
 * FULL queries of a batch (the candidate source layer), each query's reachable
 * entries are grouped into blocks of block_size consecutive entries; a block
 * scores its best member; the pool is the top_blocks best blocks under (block
 * score descending, block index ascending), except that a block still being
 * filled (the last block, when the entry count n = min(n_valid,
 * max_candidates) is not a multiple of block_size) is always in the pool and
 * takes one of its places.  Output, ready to be a REINDEX batch's lists:
 * cand_off int64 [B+1] = b * top_blocks * block_size, and cand_idx int32
 * [B][top_blocks * block_size]: the pool's entries in ascending order, then
 * -1 (a query that is not FULL gets only -1).  Scores must not be NaN.
 * 1 <= block_size <= 64, 1 <= top_blocks <= 65536; workspace from
 * csa2_candidate_pool_workspace_size. */
csa2_status csa2_candidate_pool_workspace_size(int32_t B, int32_t max_candidates, int32_t block_size,
                                               int32_t top_blocks, size_t *bytes);
csa2_status csa2_candidate_pool(int32_t B, const csa2_batch *batch, const float *scores, int64_t score_stride,
                                int32_t block_size, int32_t top_blocks, int64_t *cand_off, int32_t *cand_idx,
                                void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Compressor (Reading Notes, 3f C2 Step 1; PocketLLM page, "The compressor"):
 * n_groups groups of m consecutive tokens each become one latent.  c and g are
 * f32 [n_groups * m][d] (the tokens' latents and gate logits; g is ignored and
 * may be NULL when m == 1); per channel i of group j
 *   pooled = sum_u softmax_u(g[jm+u][i]) * c[jm+u][i],
 * then out[j] = pooled / sqrt(mean_i pooled^2 + eps) * norm_w (RMSNorm), f32
 * [n_groups][d].  fp32 arithmetic.  1 <= d <= 1024, m >= 1, eps >= 0. */
csa2_status csa2_compress(int64_t n_groups, int32_t m, int32_t d, const float *c, const float *g,
                          const float *norm_w, float eps, float *out, hipStream_t stream);

/* Compressor decode step (Reading Notes, 3f C2 Step 1: entry j is the block
 * of tokens jm .. jm + m - 1, so it exists once its last token is in;
 * PocketLLM page, "The CSA2 attention layers": the trailing partial group
 * waits in state between calls, and a step that closes no group emits
 * nothing).  One new token per sequence b at pos[b] (device int64 [B], >= 0;
 * a negative position writes and emits nothing): its latent c_new[b] and gate
 * logits g_new[b] (f32 [B][d], device) go to row u = pos[b] mod m of the
 * sequence's state kv_state[b] / score_state[b] (f32 [B][m][d], device, the
 * caller's, kept between calls; a prefill's trailing partial group is put
 * there by the caller, token p in row p mod m).  When u == m - 1 the group is
 * whole: out[b] (f32 [B][d]) becomes csa2_compress of its m rows (the same
 * bits) and emit_idx[b] (int32 [B]) = (pos[b] + 1) / m - 1, the entry's index
 * in the sequence's pool; otherwise out[b] is not written and emit_idx[b] =
 * -1.  m == 1: every step emits RMSNorm(c_new[b]) (g_new and the states are
 * not used and may be NULL).  1 <= d <= 1024. */
csa2_status csa2_compress_step(int32_t B, int32_t m, int32_t d, const int64_t *pos, const float *c_new,
                               const float *g_new, float *kv_state, float *score_state, const float *norm_w,
                               float eps, float *out, int32_t *emit_idx, hipStream_t stream);

/* Output de-rotation ("DeepSeek-V4.1-Flash on WASTE", What is new, 1. CSA2):
 * for each query b and head, the pairs of dims (rope_offset + 2i, +2i+1),
 * i < rope_dims / 2, of out [B][64][512] are rotated in place by
 * -pos[b] * inv_freq[i]:  (x, y) -> (x cos a + y sin a, -x sin a + y cos a).
 * inv_freq: f64 [rope_dims / 2] (device), the caller's frequency schedule
 * (plain RoPE theta^(-2i/rope_dims), or a YaRN-scaled one).  pos: device int64
 * [B].  Angles, sines and cosines in fp64, rounded to fp32; each output is
 * one fp32 product and one fused multiply-add (x' = fma(x, c, y s), y' =
 * fma(-x, s, y c)).  rope_dims even, at most 128. */
csa2_status csa2_derotate(const csa2_dims *dims, int32_t B, const int64_t *pos, int32_t rope_offset,
                          int32_t rope_dims, const double *inv_freq, float *out, hipStream_t stream);

/* The cache writer's quantizers (Reading Notes, 3f C4; PocketLLM page, "The
 * CSA2 attention layers" and its FP4 quantizer notes).  Both read n_rows rows
 * of d fp32 values (device) and write codes uint8 [n_rows][d/2] (element 2i in
 * the low nibble) and scales.  Codes round to the nearest E2M1 value, ties to
 * the even code, saturating at 6; a zero is stored as +0.
 *
 * FP4 main KV, one E4M3 scale per 16 values (d a multiple of 16; scales
 * [n_rows][d/16]): amax = max |x| over the block, at least 6 * 2^-9; scale =
 * e4m3(amax / 6) (the quotient in fp32, nearest-even, saturating at 448);
 * code = E2M1(x / scale), the quotient in fp32. */
csa2_status csa2_quantize_fp4_kv(int64_t n_rows, int32_t d, const float *src, uint8_t *codes,
                                 uint8_t *scales, hipStream_t stream);

/* MXFP4 index keys, one E8M0 scale per 32 values (d a multiple of 32; scales
 * [n_rows][d/32]): scale = 2^e with e = round(log2(amax / 6)) (amax / 6 in
 * fp32; e clamped to -126 .. 127, an all-zero block gets -126), stored as
 * e + 127; code = E2M1(x / 2^e). */
csa2_status csa2_quantize_mxfp4(int64_t n_rows, int32_t d, const float *src, uint8_t *codes,
                                uint8_t *scales, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
