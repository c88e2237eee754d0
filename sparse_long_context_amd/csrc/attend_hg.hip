// Two-source single-softmax attention for decode batches of fp8 / FP4 rows,
// one workgroup per (query, group of 16 heads) (Reading Notes of DeepSeek-V4.1-Flash, section
// 3f C2 Step 3; "DeepSeek-V4.1-Flash on WASTE", What is new, 1. CSA2): the
// query's heads attend, in ONE softmax, over its window rows followed by its
// selected compressed rows; every KV row is both key and value; an optional
// per-head sink logit joins only the denominator; a query with no entry gives
// zeros (PocketLLM page, "The op layer").
//
// Decode is latency-bound: few queries, 640 rows each.  So the four head
// groups of a query run as four workgroups placed eight dispatch slots apart,
// which puts them on the same XCD: the first to touch a row brings it into
// that XCD's L2 and the other three hit there.  Inside a workgroup the four
// waves (one per SIMD) split the entries, chunk by chunk (32 rows), and never
// wait for each other until the final merge:
//   S^T (32 entries x 16 heads) = K (32 x 512) * Q^T (512 x 16)
//       A operand straight from the registers the rows were loaded into,
//   online softmax in fp32 (exp2 domain, lazily raised reference),
//   O^T (512 dims x 16 heads) += V^T (512 x 32) * P^T (32 x 16)
//       A operand read transposed (ds_read_b64_tr_b16) from the wave's own
//       LDS copy of the chunk,
// all with v_mfma_f32_16x16x32_bf16.  Each wave keeps two chunks of rows in
// registers (the next one in flight while the current one is used).  At the
// end the four waves' (max, sum, O) are merged with log-sum-exp weights
// through LDS and the workgroup writes its 16 heads of the final output.
//
// The rows are FP8 (E4M3 with one UE8M0 scale per 32 values) or FP4 (E2M1
// with one E4M3 scale per 16 values, Reading Notes 3f C4), widened exactly to
// bf16 before the first product (at most 4 and 6 significant bits).  FP4 rows
// are loaded 32 dims (16 bytes) per lane at a time, so k-step s = 4a + b of
// lane group g covers dims 128a + 32g + 8b .. +7 instead of 32s + 8g .. +7;
// q is read in the same order, and each piece still lands in its natural LDS
// place for the second product.
#include "csa2_internal.h"

namespace csa2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kGroupHeads = 16;                      // heads per workgroup
constexpr int kGroups = kHeads / kGroupHeads;        // workgroups per query
constexpr int kWv = 4;                               // waves per workgroup
constexpr int kThr = 64 * kWv;
constexpr int kCh = 32;                              // entries per wave chunk
constexpr int kRowB = kDim * 2;                      // one bf16 row in LDS
constexpr int kMergeStride = kDim + 4;               // floats per head row when merging
constexpr int kRegionB = kGroupHeads * kMergeStride * 4;  // per-wave LDS region (>= 32 KiB chunk)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;  // log2 headroom before the running max is raised

static_assert(kRegionB >= kCh * kRowB, "a chunk must fit a wave's region");
static_assert(kGroups == 4, "the XCD placement assumes four head groups");

struct HgArgs {
  const int32_t* mode;
  const int64_t* win_row0;
  const int32_t* win_len;
  const int64_t* pool_row0;
  const int32_t* pool_len;
  const uint16_t* q;
  const uint8_t* win_kv;
  const uint8_t* win_scale;
  const uint8_t* comp_kv;
  const uint8_t* comp_scale;
  const int32_t* topk;
  const float* sink;
  float* out;
  float* lse;
  int32_t B;
  int32_t K;
  int32_t W;
  float scale_log2;  // softmax_scale * log2(e)
  RopeOut rope;      // de-rotation of the outputs
};

// 16-byte unit u of LDS row r sits at unit u ^ f(r), f swapping the two 2-bit
// halves of r mod 16: sixteen rows at one unit (the row-major writes) and four
// aligned rows x four aligned units (the transposing reads) both spread over
// all 16 bank groups, and f touches only the low four bits of a unit index.
__device__ __forceinline__ int swz(int r, int u) { return u ^ (((r & 3) << 2) | ((r >> 2) & 3)); }

__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint2 codes, uint32_t e) {
  // the conversion takes its scale operand's exponent field as the UE8M0
  // byte, so e = 0 (the bit pattern of +0.0f) means 2^-127 like any other
  // byte; e = 255 (NaN) is outside the format
  const float scale = __uint_as_float(e << 23);
  const auto a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, scale, false);
  const auto a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, scale, true);
  const auto a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, scale, false);
  const auto a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, scale, true);
  return make_uint4(__builtin_bit_cast(uint32_t, a0), __builtin_bit_cast(uint32_t, a1),
                    __builtin_bit_cast(uint32_t, a2), __builtin_bit_cast(uint32_t, a3));
}

// Rows of one chunk as loaded: lane (m = lane % 16, g = lane / 16) holds, for
// each of the chunk's two 16-row tiles, the 16 k-steps of 8 dims
// 32 s + 8 g .. +7 of row m of the tile: exactly the MFMA A-operand layout.
template <int KV>
struct Rows;
template <>
struct Rows<CSA2_KV_FP8_E4M3_UE8M0_32> {
  uint2 code[2][16];
  uint4 sc[2];  // the row's 16 scale bytes, one per 32 dims = one per k-step
};
template <>
struct Rows<CSA2_KV_FP4_E2M1_E4M3_16> {
  uint4 code[2][4];  // [tile][a]: codes of dims 128a + 32g .. +31
  uint32_t sw[2][4]; // [tile][a]: scale bytes 8a + 4(g/2) .. +3 (this lane's two are 8a + 2g, +1)
};

// ROPE: outputs leave de-rotated (its own instantiation)
template <int KV, bool ROPE>
__global__ __launch_bounds__(kThr) void attend_hg_kernel(HgArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kWv * kRegionB];
  __shared__ __attribute__((aligned(16))) uint8_t q_s[kGroupHeads * kRowB];  // this group's q, swizzled rows
  __shared__ int64_t ent_s[kMaxEntries];  // >= 0: window row; < 0: -(pool row) - 1
  __shared__ float ml_s[kWv][2][kGroupHeads];
  __shared__ uint32_t wcnt_s[kWv];

  // the four head groups of query b are dispatch slots 8 apart (one XCD)
  const int i = blockIdx.x;
  const int b = ((i >> 5) << 3) | (i & 7);
  const int hg = (i >> 3) & 3;
  if (b >= a.B) return;  // whole workgroup, before any barrier
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int g = lane >> 4, l16 = lane & 15;

  // ---- prologue: every global load it needs is issued before the first
  // wait -- this group's 16 q rows, the selection list, and (when it lies in
  // the window) the rows of the wave's first chunk ----
  constexpr int kQPieces = kGroupHeads * (kRowB / 16) / kThr;  // 16-byte q pieces per thread (4)
  constexpr int kListPer = kMaxTopK / kThr;                    // list entries per thread (2)
  uint4 qv[kQPieces];
#pragma unroll
  for (int it = 0; it < kQPieces; ++it) {
    const int p = t + kThr * it;
    const int h = p >> 6, u = p & 63;
    qv[it] = *reinterpret_cast<const uint4*>(a.q + ((int64_t)b * kHeads + hg * kGroupHeads + h) * kDim + 8 * u);
  }
  int wl = a.win_kv ? a.win_len[b] : 0;
  wl = wl < 0 ? 0 : (wl > a.W ? a.W : wl);
  const int64_t w0 = a.win_row0[b];
  const int md = a.mode[b];
  const bool has_list = md != CSA2_MODE_WINDOW && a.topk != nullptr && a.comp_kv != nullptr;
  int32_t idxv[kListPer];
  {
    const int32_t* lst = a.topk + (int64_t)b * a.K;
#pragma unroll
    for (int r = 0; r < kListPer; ++r) {
      const int k = r * kThr + t;
      idxv[r] = (has_list && k < a.K) ? lst[k] : -1;
    }
  }
  // ---- per-lane LDS offsets inside this wave's region ----
  // row-major write of k-step s of tile tl: wo[s & 3] + 256 (s >> 2) + 16 KiB tl
  // (the same offsets, in q_s, give this lane's q fragment of k-step s);
  // transposed read of dim tile T (16 dims) rows 4 g + tj (+16):
  // vo[T & 7] + 256 (T >> 3) (+16 KiB)
  uint8_t* region = smem + wv * kRegionB;
  const int tj = (lane >> 2) & 3, tc = lane & 3;
  const int r_lo = 4 * g + tj;
  uint32_t wo[4], vo[8];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    wo[j] = l16 * kRowB + (swz(l16, (KV == CSA2_KV_FP4_E2M1_E4M3_16) ? (4 * g + j) : (4 * j + g)) << 4);
#pragma unroll
  for (int j = 0; j < 8; ++j) vo[j] = r_lo * kRowB + (swz(r_lo, 2 * j + (tc >> 1)) << 4) + 8 * (tc & 1);

  f32x4 acc[32];
#pragma unroll
  for (int T = 0; T < 32; ++T) acc[T] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff(), l_run = 0.f;

  // entry e -> its row: window rows first (known without the list), then the
  // selected pool rows as ent_s holds them (-(row) - 1).  E counts the entries
  // known so far: the window's until the list is in.
  int E = wl;
  auto fetch = [&](int c, Rows<KV>& st) {
#pragma unroll
    for (int tl = 0; tl < 2; ++tl) {
      int e = c * kCh + 16 * tl + l16;
      if (e >= E) e = 0;  // rows past the end repeat a real row; their probability is 0
      const int64_t ev = (e < wl) ? w0 + e : ent_s[e];
      const bool pool = ev < 0;
      const int64_t row = pool ? (-ev - 1) : ev;
      if constexpr (KV == CSA2_KV_FP8_E4M3_UE8M0_32) {
        const uint8_t* rp = (pool ? a.comp_kv : a.win_kv) + row * kDim + 8 * g;
#pragma unroll
        for (int s = 0; s < 16; ++s) st.code[tl][s] = *reinterpret_cast<const uint2*>(rp + 32 * s);
        st.sc[tl] = *reinterpret_cast<const uint4*>((pool ? a.comp_scale : a.win_scale) +
                                                    row * (kDim / kScaleBlock));
      } else {
        const uint8_t* rp = (pool ? a.comp_kv : a.win_kv) + row * (kDim / 2) + 16 * g;
        const uint8_t* sp = (pool ? a.comp_scale : a.win_scale) + row * (kDim / 16) + 4 * (g >> 1);
#pragma unroll
        for (int aa = 0; aa < 4; ++aa) {
          st.code[tl][aa] = *reinterpret_cast<const uint4*>(rp + 64 * aa);
          st.sw[tl][aa] = *reinterpret_cast<const uint32_t*>(sp + 8 * aa);
        }
      }
    }
  };
  auto piece = [&](const Rows<KV>& st, int tl, int s) -> uint4 {
    if constexpr (KV == CSA2_KV_FP8_E4M3_UE8M0_32) {
      const uint32_t w = (s < 4) ? st.sc[tl].x : (s < 8) ? st.sc[tl].y : (s < 12) ? st.sc[tl].z : st.sc[tl].w;
      return fp8x8_to_bf16x8(st.code[tl][s], (w >> (8 * (s & 3))) & 0xffu);
    } else {
      const int aa = s >> 2, bb = s & 3;
      const uint4 c = st.code[tl][aa];
      const uint32_t w = (bb == 0) ? c.x : (bb == 1) ? c.y : (bb == 2) ? c.z : c.w;
      return fp4x8_e4m3_to_bf16x8(w, (st.sw[tl][aa] >> (16 * (g & 1) + 8 * (bb >> 1))) & 0xffu);
    }
  };

  // one chunk: scores from registers, rows into LDS, refill, softmax, P V
  auto consume = [&](Rows<KV>& st, int c, bool refill) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    auto qread = [&](int s) { return *reinterpret_cast<const bf16x8*>(q_s + wo[s & 3] + 256 * (s >> 2)); };
    bf16x8 qv[3] = {qread(0), qread(1), qread(2)};
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const bf16x8 qc = qv[s % 3];
      if (s + 3 < 16) qv[s % 3] = qread(s + 3);
      const uint4 k0 = piece(st, 0, s), k1 = piece(st, 1, s);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k0), qc, s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k1), qc, s1, 0, 0, 0);
      *reinterpret_cast<uint4*>(region + wo[s & 3] + 256 * (s >> 2)) = k0;
      *reinterpret_cast<uint4*>(region + wo[s & 3] + 256 * (s >> 2) + 16 * kRowB) = k1;
    }
    // the region is private to this wave and LDS serves one wave's accesses
    // in order; the fence only keeps the compiler from reordering them
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    if (refill) fetch(c + 2 * kWv, st);

    float sv[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e0 = c * kCh + 4 * g + k, e1 = e0 + 16;
      sv[k] = (e0 < E) ? s0[k] * a.scale_log2 : -__builtin_inff();
      sv[4 + k] = (e1 < E) ? s1[k] * a.scale_log2 : -__builtin_inff();
    }
    float cmax = sv[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) cmax = fmaxf(cmax, sv[k]);
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    // the reference moves only when a chunk's maximum exceeds it by more than
    // 2^kLazy, so probabilities stay below 2^kLazy and rescales are rare
    const bool raise = cmax > m_run + kLazy;  // false while both are -inf
    float alpha = 1.f;
    if (raise) {
      alpha = __builtin_amdgcn_exp2f(m_run - cmax);
      m_run = cmax;
    }
    const bool live = m_run != -__builtin_inff();
    float rs = 0.f;
    bf16x8 pb;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float pv = live ? __builtin_amdgcn_exp2f(sv[k] - m_run) : 0.f;
      rs += pv;
      pb[k] = (__bf16)pv;
    }
    rs += __shfl_xor(rs, 16);
    rs += __shfl_xor(rs, 32);
    l_run = l_run * alpha + rs;
    if (__ballot(raise)) {
#pragma unroll
      for (int T = 0; T < 32; ++T) acc[T] *= alpha;
    }
    // O^T += V^T P^T over 32 tiles of 16 dims; the transposed reads run four
    // tiles ahead of the products (one wave per SIMD: nothing else hides them)
    auto vread = [&](int T, s16x4& lo, s16x4& hi) {
      const uint8_t* pv_lo = region + vo[T & 7] + 256 * (T >> 3);
      lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((__attribute__((address_space(3))) uint8_t*)(pv_lo)));
      hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)((__attribute__((address_space(3))) uint8_t*)(pv_lo + 16 * kRowB)));
    };
    s16x4 vl[4], vh[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) vread(j, vl[j], vh[j]);
#pragma unroll
    for (int T = 0; T < 32; ++T) {
      const s16x8 v8 = {vl[T & 3][0], vl[T & 3][1], vl[T & 3][2], vl[T & 3][3],
                        vh[T & 3][0], vh[T & 3][1], vh[T & 3][2], vh[T & 3][3]};
      if (T + 4 < 32) vread(T + 4, vl[T & 3], vh[T & 3]);
      acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v8), pb, acc[T], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  };

  Rows<KV> sa, sb;
  // the wave's first chunk, when it lies in the window, goes out now
  const bool early = (wv + 1) * kCh <= wl;
  if (early) fetch(wv, sa);

  // ---- q rows into LDS (read back as the B operand: dims x heads) ----
#pragma unroll
  for (int it = 0; it < kQPieces; ++it) {
    const int p = t + kThr * it;
    const int h = p >> 6, u = p & 63;
    *reinterpret_cast<uint4*>(q_s + h * kRowB + (swz(h, u) << 4)) = qv[it];
  }
  // ---- the selected pool rows, in list order, after the window rows ----
  uint32_t nsel = 0;
  if (has_list) {
    const int32_t plen = a.pool_len[b];
    const int64_t p0 = a.pool_row0[b];
#pragma unroll
    for (int r = 0; r < kListPer; ++r) {
      if (r * kThr >= a.K) break;  // uniform
      const int32_t idx = idxv[r];
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
  E = wl + (int)nsel;
  const int nch = (E + kCh - 1) / kCh;

  // wave wv takes chunks wv, wv + 4, ... (nw of them); two register sets
  // alternate.  Inside the loop every refill is issued, even past the last
  // chunk (its rows then repeat entry 0), so each wait for a set's rows
  // leaves the other set's loads in flight.
  const int nw = (nch > wv) ? (nch - wv + kWv - 1) / kWv : 0;
  if (nw > 0) {
    if (!early) fetch(wv, sa);
    fetch(wv + kWv, sb);
    int k = 0;
#pragma clang loop unroll(disable)
    for (; k + 2 <= nw; k += 2) {
      consume(sa, wv + kWv * k, true);
      consume(sb, wv + kWv * (k + 1), true);
    }
    if (k < nw) consume(sa, wv + kWv * k, false);
  }

  // ---- merge the four waves: lane holds O[head l16][16 T + 4 g + k] ----
  float* mo = reinterpret_cast<float*>(region);
#pragma unroll
  for (int T = 0; T < 32; ++T)
    *reinterpret_cast<f32x4*>(mo + l16 * kMergeStride + 16 * T + 4 * g) = acc[T];
  if (g == 0) {
    ml_s[wv][0][l16] = m_run;
    ml_s[wv][1][l16] = l_run;
  }
  __syncthreads();
  const float* all = reinterpret_cast<const float*>(smem);
  // a thread writes the same four dims of each of its heads: their turns once
  static_assert(kThr % (kDim / 4) == 0, "a thread keeps its dims over the merge");
  Rope4 rq{1.f, 0.f, 1.f, 0.f, false, false};
  if constexpr (ROPE) rq = rope4_at(4 * (t & (kDim / 4 - 1)), a.rope.table + (int64_t)b * kRopePairs, a.rope);
#pragma unroll
  for (int j = 0; j < (kGroupHeads * kDim / 4) / kThr; ++j) {
    const int id = t + kThr * j;
    const int h = id >> 7, d4 = id & 127;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kWv; ++w) M = fmaxf(M, ml_s[w][0][h]);
    float s2 = -__builtin_inff();
    if (a.sink) {
      s2 = a.sink[hg * kGroupHeads + h] * kLog2e;
      M = fmaxf(M, s2);
    }
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.f;
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < kWv; ++w) {
        const float mw = ml_s[w][0][h];
        const float f = (mw == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        L += f * ml_s[w][1][h];
        const float4 v = *reinterpret_cast<const float4*>(all + w * (kRegionB / 4) + h * kMergeStride + 4 * d4);
        o.x += f * v.x, o.y += f * v.y, o.z += f * v.z, o.w += f * v.w;
      }
      if (a.sink) L += __builtin_amdgcn_exp2f(s2 - M);
    }
    const float inv = (L > 0.f) ? 1.f / L : 0.f;
    *reinterpret_cast<float4*>(a.out + ((int64_t)b * kHeads + hg * kGroupHeads + h) * kDim + 4 * d4) =
        rope4_apply(make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv), rq);
    if (a.lse && d4 == 0)
      a.lse[(int64_t)b * kHeads + hg * kGroupHeads + h] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
  }
}

}  // namespace

hipError_t launch_attend_hg(const csa2_dims& d, int32_t B, const csa2_batch& bt, const void* q,
                            const void* win_kv, const uint8_t* win_scale, const void* comp_kv,
                            const uint8_t* comp_scale, const int32_t* topk_idx, const float* sink, float* out,
                            float* lse, const RopeOut& rope, hipStream_t s) {
  if (d.kv_dtype == CSA2_KV_BF16) return hipErrorInvalidValue;  // bf16 rows take the all-heads kernel
  if (B == 0) return hipSuccess;
  HgArgs a;
  a.mode = bt.mode;
  a.win_row0 = bt.win_row0;
  a.win_len = bt.win_len;
  a.pool_row0 = bt.pool_row0;
  a.pool_len = bt.pool_len;
  a.q = static_cast<const uint16_t*>(q);
  a.win_kv = static_cast<const uint8_t*>(win_kv);
  a.win_scale = win_scale;
  a.comp_kv = static_cast<const uint8_t*>(comp_kv);
  a.comp_scale = comp_scale;
  a.topk = topk_idx;
  a.sink = sink;
  a.out = out;
  a.lse = lse;
  a.B = B;
  a.K = d.index_topk;
  a.W = d.window;
  a.scale_log2 = d.softmax_scale * kLog2e;
  a.rope = rope;
  // 32 workgroups per 8 queries: slot i -> query 8 (i / 32) + i % 8, head group (i / 8) % 4
  const dim3 grid((unsigned)(32 * ((B + 7) / 8)));
  const bool turn = rope.table != nullptr;
  if (d.kv_dtype == CSA2_KV_FP8_E4M3_UE8M0_32) {
    if (turn) hipLaunchKernelGGL((attend_hg_kernel<CSA2_KV_FP8_E4M3_UE8M0_32, true>), grid, dim3(kThr), 0, s, a);
    else hipLaunchKernelGGL((attend_hg_kernel<CSA2_KV_FP8_E4M3_UE8M0_32, false>), grid, dim3(kThr), 0, s, a);
  } else {
    if (turn) hipLaunchKernelGGL((attend_hg_kernel<CSA2_KV_FP4_E2M1_E4M3_16, true>), grid, dim3(kThr), 0, s, a);
    else hipLaunchKernelGGL((attend_hg_kernel<CSA2_KV_FP4_E2M1_E4M3_16, false>), grid, dim3(kThr), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace csa2
