// Two-source single-softmax attention for batches of many queries with bf16
// KV (a prefill chunk, or a decode batch of a few hundred queries), one
// workgroup of four waves per query (Reading Notes of DeepSeek-V4.1-Flash,
// section 3f C2 Step 3; "DeepSeek-V4.1-Flash on WASTE", What is new, 1. CSA2):
// the query's 64 heads attend, in ONE softmax, over its window rows followed
// by its selected compressed rows; every KV row is both key and value; an
// optional per-head sink logit joins only the denominator; a query with no
// entry gives zeros (PocketLLM page, "The op layer").
//
// Rows reach LDS by DMA (global_load_lds_dwordx4: lane l's 16 bytes land at
// the instruction's LDS base + 16 l), into a ring of four 32-row slots, so
// three chunks are in flight without holding a register.  Each of the four
// waves gathers 8 rows of a chunk, one whole 1 KiB row per instruction; lane
// l fetches 16-byte unit l ^ f(r) of row r, which leaves the slot XOR-swizzled.
//
// Wave w = hh + 2 dh (one per SIMD) owns heads 32 hh .. +31 and dims
// 256 dh .. +255.  Per chunk of 32 entries:
//   S^T (32 entries x 32 heads) = K (32 x 256) * Q^T (256 x 32)
//       K fragments read from the slot, Q^T held in registers for the query;
//   the two dim halves' partial scores are added through LDS (in the same
//   order in both waves, so both hold the same scores), online softmax in
//   fp32 (exp2 domain, lazily raised reference);
//   O^T (256 dims x 32 heads) += V^T (256 x 32) * P^T (32 x 32)
//       V^T read transposed (ds_read_b64_tr_b16) from the same slot.
// All products are v_mfma_f32_16x16x32_bf16 with their accumulators in the
// accumulation registers.  Per entry a CU moves 1 KiB into LDS, reads 2 KiB
// of K and 2 KiB of V^T out of it and exchanges 256 B of partial scores; the
// K and V^T of each dim half are read by the two head halves.
//
// Workgroup i runs on XCD i mod 8 (round-robin dispatch); queries are handed
// out so each XCD takes a contiguous run, which keeps the window rows that
// consecutive prefill queries share (127 of 128) in that XCD's L2.
#include "csa2_internal.h"

namespace csa2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void global_cvoid;

constexpr int kWv = 4;
constexpr int kThr = 64 * kWv;
constexpr int kCh = 32;                 // entries per chunk
constexpr int kRowB = kDim * 2;         // one bf16 row
constexpr int kSlotB = kCh * kRowB;     // 32 KiB per ring slot
constexpr int kSlots = 4;               // chunk c lives in slot c % 4
constexpr int kRowsPerWave = kCh / kWv; // rows of a chunk each wave gathers
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;  // log2 headroom before the running max is raised

struct MqArgs {
  const int32_t* mode;
  const int64_t* win_row0;
  const int32_t* win_len;
  const int64_t* pool_row0;
  const int32_t* pool_len;
  const uint16_t* q;
  const uint8_t* win_kv;
  const uint8_t* comp_kv;
  const int32_t* topk;
  const float* sink;
  float* out;
  float* lse;
  float* part_o;   // [B][S][64][512] unnormalised partial outputs (entry splits only)
  float* part_ml;  // [B][S][64][2]   running max (log2 units) and sum
  int32_t n_split;
  int32_t B;
  int32_t K;
  int32_t W;
  float scale_log2;  // softmax_scale * log2(e)
};

// 16-byte unit u of a slot row r sits at unit u ^ f(r), f swapping the two
// 2-bit halves of r mod 16: sixteen rows at one unit (the K fragment reads)
// and four aligned rows x four aligned units (the transposing reads) both
// spread over all 16 bank groups; f touches only the low four bits of u.
__device__ __forceinline__ int swz(int r, int u) { return u ^ (((r & 3) << 2) | ((r >> 2) & 3)); }

// s_waitcnt with only the vector-memory count constrained (expcnt and lgkmcnt
// at their maxima): vmcnt in bits 3:0 and 15:14.
#define CSA2_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | 0x0F70)

__global__ __launch_bounds__(kThr) void attend_mq_kernel(MqArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kSlots * kSlotB];
  __shared__ __attribute__((aligned(16))) f32x4 xs[kWv][4][64];  // partial scores, one chunk at a time
  __shared__ int64_t ent_s[kMaxEntries];  // >= 0: window row; < 0: -(pool row) - 1
  __shared__ uint32_t wcnt_s[kWv];

  // contiguous runs of (query, split) pairs per XCD: workgroup i -> XCD
  // i % 8, slot i / 8
  const int nwg = (int)gridDim.x;
  const int xcd = (int)blockIdx.x & 7, wslot = (int)blockIdx.x >> 3;
  const int per = nwg >> 3, rem = nwg & 7;
  const int item = xcd * per + (xcd < rem ? xcd : rem) + wslot;
  const int b = item / a.n_split, sp = item % a.n_split;
  if (b >= a.B) return;  // whole workgroup, before any barrier
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int hh = wv & 1, dh = wv >> 1;

  // ---- Q^T fragments: head 32 hh + 16 ht + l16, dims 256 dh + 32 s + 8 g .. +7 ----
  bf16x8 qf[2][8];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const uint16_t* qp = a.q + ((int64_t)b * kHeads + 32 * hh + 16 * ht + l16) * kDim + 256 * dh + 8 * g;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[ht][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 32 * s));
  }

  // ---- entry list: window rows, then the selected pool rows in list order ----
  int wl = a.win_kv ? a.win_len[b] : 0;
  wl = wl < 0 ? 0 : (wl > a.W ? a.W : wl);
  const int64_t w0 = a.win_row0[b];
  for (int e = t; e < wl; e += kThr) ent_s[e] = w0 + e;
  const int md = a.mode[b];
  uint32_t nsel = 0;
  if (md != CSA2_MODE_WINDOW && a.topk != nullptr && a.comp_kv != nullptr) {
    const int32_t plen = a.pool_len[b];
    const int64_t p0 = a.pool_row0[b];
    const int32_t* lst = a.topk + (int64_t)b * a.K;
    for (int r0 = 0; r0 < a.K; r0 += kThr) {
      const int k = r0 + t;
      const int32_t idx = (k < a.K) ? lst[k] : -1;
      const bool ok = (idx >= 0) & (idx < plen);
      const uint64_t m = __ballot(ok);
      if (lane == 0) wcnt_s[wv] = __popcll(m);
      __syncthreads();
      uint32_t before = nsel, tot = 0;
#pragma unroll
      for (int w = 0; w < kWv; ++w) {
        before += (w < wv) ? wcnt_s[w] : 0u;
        tot += wcnt_s[w];
      }
      before += __popcll(m & ((1ull << lane) - 1ull));
      if (ok) ent_s[wl + before] = -(p0 + idx) - 1;
      nsel += tot;
      __syncthreads();
    }
  }
  __syncthreads();
  const int E = wl + (int)nsel;
  // this workgroup's chunks: [c_beg, c_beg + nch) of the query's
  const int nch_all = (E + kCh - 1) / kCh;
  const int cps = (nch_all + a.n_split - 1) / a.n_split;
  const int c_beg = sp * cps;
  const int c_end = c_beg + cps < nch_all ? c_beg + cps : nch_all;
  const int nch = c_end > c_beg ? c_end - c_beg : 0;  // local chunk c is the query's c_beg + c

  // ---- gather of chunk c into its slot: this wave's 8 rows, one DMA each;
  // rows past the last entry repeat entry 0 (their probability is 0).  Lane
  // i < 8 looks up the entry of row i ahead of time (entry_for); the DMAs
  // then take each row from that lane, so no LDS round trip sits between
  // them ----
  auto entry_for = [&](int c) __attribute__((always_inline)) -> int64_t {
    int e = (c_beg + c) * kCh + kRowsPerWave * wv + (lane & (kRowsPerWave - 1));
    if (e >= E) e = 0;
    return ent_s[e];
  };
  auto gather = [&](int c, int64_t evl) __attribute__((always_inline)) {
    uint8_t* slot = ring + (c % kSlots) * kSlotB;
    const uint32_t lo = (uint32_t)evl, hi = (uint32_t)((uint64_t)evl >> 32);
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int r = kRowsPerWave * wv + i;
      const int64_t ev = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, i) << 32) |
                                   (uint32_t)__builtin_amdgcn_readlane((int)lo, i));
      const uint8_t* src = (ev < 0) ? a.comp_kv + (-ev - 1) * kRowB : a.win_kv + ev * kRowB;
      __builtin_amdgcn_global_load_lds((global_cvoid*)(src + (swz(r, lane) << 4)),
                                       (lds_void*)(slot + r * kRowB), 16, 0, 0);
    }
  };

  // ---- per-lane LDS offsets within a slot ----
  // K fragment (entry tile et, k-step s): row 16 et + l16, unit 32 dh + 4 s + g
  //   -> ko[s & 3] + 256 (s >> 2) (+16 KiB for et = 1);
  // V^T of dim tile dt (16 dims), rows 4 g + tj (+16): vo[dt & 7] + 256 (dt >> 3) (+16 KiB)
  const int tj = (lane >> 2) & 3, tc = lane & 3;
  const int r_lo = 4 * g + tj;
  uint32_t ko[4], vo[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) ko[j] = l16 * kRowB + 512 * dh + (swz(l16, 4 * j + g) << 4);
#pragma unroll
  for (int j = 0; j < 8; ++j) vo[j] = r_lo * kRowB + 512 * dh + (swz(r_lo, 2 * j + (tc >> 1)) << 4) + 8 * (tc & 1);

  f32x4 acc[16][2];  // O^T tiles: [dim tile][head tile]
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) acc[dt][0] = acc[dt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  // running reference (log2 units) of the lane's two heads, the same in the
  // four lanes of a head; the sums are this lane's share (reduced at the end)
  float m_run[2] = {-__builtin_inff(), -__builtin_inff()}, l_run[2] = {0.f, 0.f};

  // maximum / sum over the four lanes of a head (lanes l16 + 16 g): swap with
  // the lane 32 away, then with the lane 16 away (gfx950 permlane swaps)
  auto head_max = [&](float x) __attribute__((always_inline)) -> float {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    const auto r2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r2[0]), __uint_as_float(r2[1]));
  };
  auto head_sum = [&](float x) __attribute__((always_inline)) -> float {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const auto r2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
  };

  // Chunk c: QK from slot c % 4, partial-score exchange (two barriers: one
  // after the writes, one after the reads, so one buffer serves every chunk),
  // the gather of chunk c + 3 into the slot chunk c - 1 used (every wave has
  // finished with it by the first barrier), softmax, PV from slot c % 4.
  // Chunk c + 1 must have landed before the second barrier: each wave waits
  // for its own DMAs of c + 1 (issued two chunks earlier; those of c + 2 stay
  // in flight).
  auto step = [&](int c) __attribute__((always_inline)) {
    const uint8_t* slot = ring + (c % kSlots) * kSlotB;
    const int64_t ev_next = entry_for(c + 3);  // its LDS latency hides behind QK
    f32x4 sa[2][2];  // [entry tile][head tile]
#pragma unroll
    for (int et = 0; et < 2; ++et) sa[et][0] = sa[et][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint32_t o = ko[s & 3] + 256 * (s >> 2);
      const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(slot + o);
      const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(slot + o + 16 * kRowB);
      sa[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[0][s], sa[0][0], 0, 0, 0);
      sa[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[1][s], sa[0][1], 0, 0, 0);
      sa[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[0][s], sa[1][0], 0, 0, 0);
      sa[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[1][s], sa[1][1], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) xs[wv][i][lane] = sa[i >> 1][i & 1];
    __syncthreads();
    f32x4 o4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o4[i] = xs[wv ^ 2][i][lane];
    if (c + 2 < nch) CSA2_WAIT_VMCNT(kRowsPerWave); else CSA2_WAIT_VMCNT(0);
    __syncthreads();
    if (c + 3 < nch) gather(c + 3, ev_next);

    // full scores: the dim-0 half's partial plus the dim-1 half's, in that order
    float sv[2][8];  // [head tile][entry 4 g + k, then 16 + 4 g + k]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int et = i >> 1, ht = i & 1;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float s2 = dh ? o4[i][k] + sa[et][ht][k] : sa[et][ht][k] + o4[i][k];
        const int e = (c_beg + c) * kCh + 16 * et + 4 * g + k;
        sv[ht][4 * et + k] = (e < E) ? s2 * a.scale_log2 : -__builtin_inff();
      }
    }
    // The reference of a head moves only when one of its scores exceeds it by
    // more than 2^kLazy, so probabilities stay below 2^kLazy.  Each lane tests
    // its own scores; only when some lane would move does the wave reduce the
    // chunk maxima over each head's four lanes and rescale.
    float lm[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      lm[ht] = sv[ht][0];
#pragma unroll
      for (int k = 1; k < 8; ++k) lm[ht] = fmaxf(lm[ht], sv[ht][k]);
    }
    if (__ballot((lm[0] > m_run[0] + kLazy) || (lm[1] > m_run[1] + kLazy))) {
      float alpha[2];
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const float cmax = head_max(lm[ht]);
        alpha[ht] = 1.f;
        if (cmax > m_run[ht] + kLazy) {  // false while both are -inf
          alpha[ht] = __builtin_amdgcn_exp2f(m_run[ht] - cmax);
          m_run[ht] = cmax;
        }
        l_run[ht] *= alpha[ht];
      }
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) acc[dt][0] *= alpha[0], acc[dt][1] *= alpha[1];
    }
    // every chunk holds at least one entry, so after the first the references
    // are finite
    bf16x8 pb[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      float rs = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float pv = __builtin_amdgcn_exp2f(sv[ht][k] - m_run[ht]);
        rs += pv;
        pb[ht][k] = (__bf16)pv;
      }
      l_run[ht] += rs;
    }

    // O^T += V^T P^T over 16 dim tiles; transposed reads run two tiles ahead
    auto vread = [&](int dt, s16x4& lo, s16x4& hi) __attribute__((always_inline)) {
      const uint8_t* p = slot + vo[dt & 7] + 256 * (dt >> 3);
      lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((__attribute__((address_space(3))) uint8_t*)(p)));
      hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)((__attribute__((address_space(3))) uint8_t*)(p + 16 * kRowB)));
    };
    s16x4 vl[2], vh[2];
    vread(0, vl[0], vh[0]);
    vread(1, vl[1], vh[1]);
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
      const s16x8 v8 = {vl[dt & 1][0], vl[dt & 1][1], vl[dt & 1][2], vl[dt & 1][3],
                        vh[dt & 1][0], vh[dt & 1][1], vh[dt & 1][2], vh[dt & 1][3]};
      if (dt + 2 < 16) vread(dt + 2, vl[dt & 1], vh[dt & 1]);
      acc[dt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v8), pb[0], acc[dt][0], 0, 0, 0);
      acc[dt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v8), pb[1], acc[dt][1], 0, 0, 0);
    }
  };

  if (nch > 0) {
    // chunks 0, 1, 2 in flight; chunk 0 landed everywhere before the first step
#pragma unroll
    for (int c = 0; c < 3; ++c)
      if (c < nch) gather(c, entry_for(c));
    if (nch > 2) CSA2_WAIT_VMCNT(2 * kRowsPerWave);
    else CSA2_WAIT_VMCNT(0);
    __syncthreads();
#pragma clang loop unroll(disable)
    for (int c = 0; c < nch; ++c) step(c);
  }

  // ---- epilogue: lane holds O^T[256 dh + 16 dt + 4 g + k][32 hh + 16 ht + l16] ----
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const int head = 32 * hh + 16 * ht + l16;
    const float lsum = head_sum(l_run[ht]);
    if (a.n_split > 1) {  // unnormalised partials, merged by attend_combine
      const int64_t pslot = ((int64_t)b * a.n_split + sp) * kHeads + head;
      float* op = a.part_o + pslot * kDim + 256 * dh + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 16; ++dt)
        *reinterpret_cast<float4*>(op + 16 * dt) =
            make_float4(acc[dt][ht][0], acc[dt][ht][1], acc[dt][ht][2], acc[dt][ht][3]);
      if (g == 0 && dh == 0) {
        a.part_ml[pslot * 2] = m_run[ht];
        a.part_ml[pslot * 2 + 1] = lsum;
      }
      continue;
    }
    float M = m_run[ht], L = lsum, f;
    if (a.sink) {
      const float s2 = a.sink[head] * kLog2e;
      const float M2 = fmaxf(M, s2);
      L = L * __builtin_amdgcn_exp2f(M - M2) + __builtin_amdgcn_exp2f(s2 - M2);
      f = __builtin_amdgcn_exp2f(M - M2) / L;
      M = M2;
    } else {
      f = (L > 0.f) ? 1.f / L : 0.f;
    }
    float* op = a.out + ((int64_t)b * kHeads + head) * kDim + 256 * dh + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
      const f32x4 v = acc[dt][ht] * f;
      *reinterpret_cast<float4*>(op + 16 * dt) = make_float4(v[0], v[1], v[2], v[3]);
    }
    if (a.lse && g == 0 && dh == 0)
      a.lse[(int64_t)b * kHeads + head] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
  }
}

}  // namespace

hipError_t launch_attend_mq(const csa2_dims& d, int32_t B, const csa2_batch& bt, const void* q,
                            const void* win_kv, const void* comp_kv, const int32_t* topk_idx, const float* sink,
                            float* out, float* lse, int n_split, float* partial, hipStream_t s) {
  if (B == 0) return hipSuccess;
  MqArgs a;
  a.mode = bt.mode;
  a.win_row0 = bt.win_row0;
  a.win_len = bt.win_len;
  a.pool_row0 = bt.pool_row0;
  a.pool_len = bt.pool_len;
  a.q = static_cast<const uint16_t*>(q);
  a.win_kv = static_cast<const uint8_t*>(win_kv);
  a.comp_kv = static_cast<const uint8_t*>(comp_kv);
  a.topk = topk_idx;
  a.sink = sink;
  a.out = out;
  a.lse = lse;
  if (n_split < 1) n_split = 1;
  a.n_split = n_split;
  a.part_o = partial;
  a.part_ml = partial ? partial + (size_t)B * n_split * kHeads * kDim : nullptr;
  a.B = B;
  a.K = d.index_topk;
  a.W = d.window;
  a.scale_log2 = d.softmax_scale * kLog2e;
  hipLaunchKernelGGL(attend_mq_kernel, dim3((unsigned)(B * n_split)), dim3(kThr), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_split == 1) return e;
  return launch_attend_combine(B, n_split, a.part_o, a.part_ml, sink, out, lse, s);
}

}  // namespace csa2
