// CSA2_TRACE=1: per-stage checksums of what csa2_decode, csa2_decode_static
// and csa2_prefill computed, one line per stage on stderr, in the format the
// oracle's trace uses for the same results, so a divergence can be located
// by comparing the two line by line.  Each line waits for the stage on its
// stream and copies its output to the host: a debugging aid, never a fast
// path.
//
//   csa2-trace <call> scores finite=<n> sum=<s>          finite scores of the
//       Full / Reindex queries' candidates, summed in fp64 query by query in
//       candidate order (exact: the scores are the oracle's bits)
//   csa2-trace <call> topk rows=<r> chosen=<c> fnv1a=<h>  the top-K rows the
//       call wrote: count of entries >= 0 and the 64-bit FNV-1a hash of the
//       rows' int32 values (little-endian), row by row
//   csa2-trace <call> attend out_sum=<s> out_abs=<a> lse_sum=<l> lse_ninf=<k>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "csa2_internal.h"

namespace csa2 {
namespace {

template <typename T>
bool fetch(std::vector<T>& h, const T* d, size_t n) {
  h.resize(n);
  if (n == 0) return true;
  if (!d) return false;
  return hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost) == hipSuccess;
}

struct HostBatch {
  std::vector<int64_t> pos, cand_off;
  std::vector<int32_t> mode, ratio, pool_len;
};

bool fetch_batch(HostBatch& hb, int32_t B, const csa2_batch& bt) {
  bool ok = fetch(hb.pos, bt.pos, B) && fetch(hb.mode, bt.mode, B) && fetch(hb.ratio, bt.compress_ratio, B) &&
            fetch(hb.pool_len, bt.pool_len, B);
  if (ok && bt.cand_off) ok = fetch(hb.cand_off, bt.cand_off, (size_t)B + 1);
  return ok;
}

bool selects(int md) { return md == CSA2_MODE_FULL || md == CSA2_MODE_REINDEX; }

// candidates query b scores (the same count the index kernels use)
int64_t cand_count(const HostBatch& hb, const csa2_batch& bt, int b) {
  const int md = hb.mode[b];
  if (!selects(md)) return 0;
  int64_t nv = 0;
  const int32_t m = hb.ratio[b];
  if (m > 0 && hb.pos[b] >= 0) nv = std::min<int64_t>((hb.pos[b] + 1) / m, hb.pool_len[b]);
  int64_t n = (md == CSA2_MODE_FULL) ? nv : (bt.cand_off ? hb.cand_off[b + 1] - hb.cand_off[b] : 0);
  return std::min<int64_t>(n, bt.max_candidates);
}

void fail(const char* call, const char* stage) { fprintf(stderr, "csa2-trace %s %s unavailable\n", call, stage); }

}  // namespace

bool trace_enabled() {
  const char* e = getenv("CSA2_TRACE");
  return e && e[0] == '1' && e[1] == '\0';
}

void trace_scores(const char* call, int32_t B, const csa2_batch& bt, const float* scores, int64_t stride,
                  hipStream_t s) {
  HostBatch hb;
  std::vector<float> sc;
  if (hipStreamSynchronize(s) != hipSuccess || !fetch_batch(hb, B, bt) ||
      !fetch(sc, scores, (size_t)B * (size_t)stride)) {
    fail(call, "scores");
    return;
  }
  int64_t finite = 0;
  double sum = 0.0;
  for (int b = 0; b < B; ++b) {
    const int64_t n = cand_count(hb, bt, b);
    for (int64_t j = 0; j < n; ++j) {
      const float v = sc[(size_t)b * (size_t)stride + (size_t)j];
      if (isfinite(v)) ++finite, sum += (double)v;
    }
  }
  fprintf(stderr, "csa2-trace %s scores finite=%lld sum=%.17g\n", call, (long long)finite, sum);
}

void trace_topk(const char* call, int32_t B, const csa2_batch& bt, int32_t K, const int32_t* topk, hipStream_t s) {
  HostBatch hb;
  std::vector<int32_t> sel;
  if (hipStreamSynchronize(s) != hipSuccess || !fetch_batch(hb, B, bt) || !fetch(sel, topk, (size_t)B * K)) {
    fail(call, "topk");
    return;
  }
  uint64_t h = 0xcbf29ce484222325ull;
  int64_t rows = 0, chosen = 0;
  for (int b = 0; b < B; ++b) {
    if (!selects(hb.mode[b])) continue;
    ++rows;
    for (int i = 0; i < K; ++i) {
      const uint32_t v = (uint32_t)sel[(size_t)b * K + i];
      chosen += sel[(size_t)b * K + i] >= 0;
      for (int k = 0; k < 4; ++k) h = (h ^ ((v >> (8 * k)) & 0xFFu)) * 0x100000001b3ull;
    }
  }
  fprintf(stderr, "csa2-trace %s topk rows=%lld chosen=%lld fnv1a=%016llx\n", call, (long long)rows,
          (long long)chosen, (unsigned long long)h);
}

void trace_attend(const char* call, int32_t B, const float* out, const float* lse, hipStream_t s) {
  std::vector<float> o, l;
  if (hipStreamSynchronize(s) != hipSuccess || !fetch(o, out, (size_t)B * kHeads * kDim) ||
      (lse && !fetch(l, lse, (size_t)B * kHeads))) {
    fail(call, "attend");
    return;
  }
  double os = 0.0, oa = 0.0, ls = 0.0;
  int64_t ninf = 0;
  for (float v : o) os += (double)v, oa += fabs((double)v);
  for (float v : l) {
    if (isfinite(v)) ls += (double)v;
    else ++ninf;
  }
  fprintf(stderr, "csa2-trace %s attend out_sum=%.6e out_abs=%.6e lse_sum=%.6e lse_ninf=%lld\n", call, os, oa, ls,
          (long long)ninf);
}

}  // namespace csa2
