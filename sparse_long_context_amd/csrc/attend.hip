// Two-source single-softmax attention (Reading Notes of DeepSeek-V4.1-Flash,
// section 3f C2 Step 3; "DeepSeek-V4.1-Flash on WASTE", What is new, 1. CSA2):
// each query's 64 heads attend, in ONE softmax, over its window rows followed
// by its selected compressed rows.  Every KV row (512 dims) serves all heads
// as both key and value.  An optional per-head sink logit joins only the
// denominator; a query with no entry yields zeros (PocketLLM page, "The op
// layer").
//
// This kernel serves rows stored narrower than bf16 (fp8, FP4): decode
// batches of more than 64 queries and prefill chunks of any length; bf16
// rows go to the DMA-ring kernel.
//
// Workgroup = one (query, split) pair, 8 waves, two per SIMD so one wave's
// latency (LDS, softmax, barriers) hides behind another's matrix work.  Wave w
// owns heads 16(w%4) .. +15 and half h = w/4 of the 512 dims: it contracts its
// dim half of q.k, the two halves add their partial scores through LDS (a + b
// is the same sum in both waves), and it accumulates its dim half of the
// output.  Entries are processed in chunks of 32 rows staged in LDS (double
// buffered); their global loads are issued two chunks ahead into registers,
// and fp8 rows are widened to bf16 on the way into LDS.  Per chunk and wave:
//   S^T (32 entries x 16 heads) = K (32 x 256) * Q^T (256 x 16)   v_mfma_f32_16x16x32_bf16
//   + the partner half's partial, online softmax in fp32 (exp2 domain)
//   O^T (256 dims x 16 heads) += V^T (256 x 32) * P^T (32 x 16)     same MFMA
// Putting the entries on the M side of the first product leaves each lane's
// probabilities (head = lane % 16, 8 entries) exactly where the second
// product's B operand needs them.  V^T fragments come straight out of the
// row-major LDS tile with the gfx950 transposing LDS read (ds_read_b64_tr_b16).
// Rows are XOR-swizzled in 16-byte units so the row reads of the first product
// and the transposed reads of the second both spread over all LDS banks.
//
// FP8 rows (E4M3 with one UE8M0 scale per 32 values) and FP4 rows (E2M1 with
// one E4M3 scale per 16 values) are widened to bf16 while staging, exactly
// (each product has at most 4 and 6 significant bits).
#include "csa2_internal.h"

namespace csa2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kChunk = 32;                         // entries per staged chunk
constexpr int kRowBytes = kDim * 2;                // one bf16 row in LDS
constexpr int kBufBytes = kChunk * kRowBytes;      // 32 KiB per buffer
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;  // log2 headroom before the running max is raised

struct AttendArgs {
  const int64_t* pos;
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
  float* part_o;   // [B][S][64][512] unnormalised partial outputs (split only)
  float* part_ml;  // [B][S][64][2]   running max (log2 units) and sum
  int32_t K;
  int32_t W;
  int32_t n_split;
  float scale_log2;  // softmax_scale * log2(e)
  RopeOut rope;      // de-rotation of unsplit outputs (splits: the merge's)
};

// 16-byte unit u of LDS row r lives at unit u ^ f(r), where f swaps the two
// 2-bit halves of r mod 16 (so f(r) = f(r + 16)).  Sixteen consecutive rows at
// one unit (the row reads of the first product), and four aligned rows x four
// aligned units (the transposing reads of the second), both land on 16
// distinct bank groups.  f touches only the low four bits of a unit index, so
// every fragment address is a per-lane base plus a compile-time offset.
__device__ __forceinline__ int swz_unit(int r, int u) { return u ^ (((r & 3) << 2) | ((r >> 2) & 3)); }
__device__ __forceinline__ int lds_off(int r, int byte) {
  return r * kRowBytes + (swz_unit(r, byte >> 4) << 4) + (byte & 15);
}

// Widen 8 E4M3 codes (two dwords) times 2^(e - 127) to 8 bf16 with the gfx950
// scaled conversion; exact, since each product has at most 4 significant bits.
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

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kPieces = kBufBytes / 16 / kThreads;  // 16-byte LDS units per thread per chunk (4)

// ROPE: unsplit outputs leave de-rotated (its own instantiation)
template <int KV, bool ROPE>
__global__ __launch_bounds__(kThreads) void attend_kernel(AttendArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kBufBytes];  // double buffer
  __shared__ __attribute__((aligned(16))) float xs_s[kWaves][8][64];     // partial scores
  __shared__ int64_t ent_s[kMaxEntries];  // >= 0: window row; < 0: -(pool row) - 1
  __shared__ uint32_t wcnt_s[kWaves];

  const int b = blockIdx.x / a.n_split;
  const int sp = blockIdx.x % a.n_split;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int hg = wv & 3, dh = wv >> 2;  // head group, dim half
  const int g = lane >> 4, l16 = lane & 15;

  // ---- entry list: window rows, then the selected pool rows in list order ----
  int wl = a.win_kv ? a.win_len[b] : 0;  // no window rows without a window source
  wl = wl < 0 ? 0 : (wl > a.W ? a.W : wl);
  const int64_t w0 = a.win_row0[b];
  for (int e = t; e < wl; e += kThreads) ent_s[e] = w0 + e;
  const int md = a.mode[b];
  uint32_t nsel = 0;
  if (md != CSA2_MODE_WINDOW && a.topk != nullptr && a.comp_kv != nullptr) {
    const int32_t plen = a.pool_len[b];
    const int64_t p0 = a.pool_row0[b];
    const int32_t* lst = a.topk + (int64_t)b * a.K;
    for (int r0 = 0; r0 < a.K; r0 += kThreads) {
      const int i = r0 + t;
      const int32_t idx = (i < a.K) ? lst[i] : -1;
      const bool ok = (idx >= 0) & (idx < plen);
      const uint64_t m = __ballot(ok);
      if (lane == 0) wcnt_s[wv] = __popcll(m);
      __syncthreads();
      uint32_t before = nsel, tot = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
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
  const int nch = (E + kChunk - 1) / kChunk;
  const int cps = (nch + a.n_split - 1) / a.n_split;
  const int cbeg = sp * cps;
  const int cend = (cbeg + cps < nch) ? cbeg + cps : nch;

  // ---- q fragments of this wave's 16 heads and dim half (B operand, dims x heads) ----
  const int head = hg * 16 + l16;
  bf16x8 qf[8];
  {
    const uint16_t* qp = a.q + ((int64_t)b * kHeads + head) * kDim + dh * 256 + g * 8;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + kk * 32));
  }

  // ---- per-lane LDS bases: K fragment kk = 4a + bq of row l16 sits at
  // qo[bq] + 512 dh + 256 a; V^T tile tt = 8a + bt of rows 4g + tj at
  // vo[bt] + 512 dh + 256 a; rows r + 16 are 16 KiB further on ----
  const int tj = (lane >> 2) & 3, tc = lane & 3;
  const int r_lo = 4 * g + tj;
  uint32_t qo[4], vo[8];
#pragma unroll
  for (int bq = 0; bq < 4; ++bq) qo[bq] = l16 * kRowBytes + dh * 512 + (swz_unit(l16, 4 * bq + g) << 4);
#pragma unroll
  for (int bt = 0; bt < 8; ++bt)
    vo[bt] = r_lo * kRowBytes + dh * 512 + (swz_unit(r_lo, 2 * bt + (tc >> 1)) << 4) + 8 * (tc & 1);

  f32x4 acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff(), l_run = 0.f;

  // ---- one chunk of 32 staged rows ----
  auto consume = [&](const uint8_t* base, int c) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const uint8_t* pk = base + qo[kk & 3] + 256 * (kk >> 2);
      const uint4 k0 = *reinterpret_cast<const uint4*>(pk);
      const uint4 k1 = *reinterpret_cast<const uint4*>(pk + 16 * kRowBytes);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k0), qf[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k1), qf[kk], s1, 0, 0, 0);
    }
    // add the partner half's partial scores (same sum, same order of the two terms)
    float* mine = &xs_s[wv][0][0];
#pragma unroll
    for (int i = 0; i < 4; ++i) mine[i * 64 + lane] = s0[i], mine[(4 + i) * 64 + lane] = s1[i];
    __syncthreads();
    const float* other = &xs_s[wv ^ 4][0][0];
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float t0 = (dh == 0) ? s0[i] + other[i * 64 + lane] : other[i * 64 + lane] + s0[i];
      const float t1 = (dh == 0) ? s1[i] + other[(4 + i) * 64 + lane] : other[(4 + i) * 64 + lane] + s1[i];
      const int e0 = c * kChunk + 4 * g + i, e1 = e0 + 16;
      sv[i] = (e0 < E) ? t0 * a.scale_log2 : -__builtin_inff();
      sv[4 + i] = (e1 < E) ? t1 * a.scale_log2 : -__builtin_inff();
    }
    float cmax = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) cmax = fmaxf(cmax, sv[i]);
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    // The running reference moves only when a chunk's maximum exceeds it by
    // more than 2^kLazy: until then probabilities stay below 2^kLazy (no
    // overflow risk in fp32 or bf16) and the accumulators need no rescale.
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
    for (int i = 0; i < 8; ++i) {
      const float pv = live ? __builtin_amdgcn_exp2f(sv[i] - m_run) : 0.f;
      rs += pv;
      pb[i] = (__bf16)pv;
    }
    rs += __shfl_xor(rs, 16);
    rs += __shfl_xor(rs, 32);
    l_run = l_run * alpha + rs;
    if (__ballot(raise)) {  // wave-uniform: rescale only when some head moved
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) acc[tt] *= alpha;
    }
    // O^T (this wave's 256 dims x 16 heads) += V^T P^T, 16 tiles of 16 dims
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      const uint8_t* pv_lo = base + vo[tt & 7] + 256 * (tt >> 3);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)((__attribute__((address_space(3))) uint8_t*)(pv_lo)));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)((__attribute__((address_space(3))) uint8_t*)(pv_lo + 16 * kRowBytes)));
      typedef short s16x8 __attribute__((ext_vector_type(8)));
      const s16x8 v8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v8), pb, acc[tt], 0, 0, 0);
    }
  };

  // ---- staging: chunk c's rows travel HBM -> registers -> LDS.  Two register
  // sets alternate, so while chunk c is consumed the loads of chunks c+1 and
  // c+2 are in flight; LDS is double buffered.  A wave instruction moves half a
  // 1 KiB bf16 row; rows past the last entry repeat a real row (probability 0).
  struct Stage {
    uint2 code[KV == CSA2_KV_FP8_E4M3_UE8M0_32 ? kPieces : 1];
    uint32_t c4[KV == CSA2_KV_FP4_E2M1_E4M3_16 ? kPieces : 1];
    uint32_t sc[kPieces];
  };
  auto fetch = [&](int c, Stage& st) {
#pragma unroll
    for (int it = 0; it < kPieces; ++it) {
      const int p = it * kThreads + t;
      const int er = p >> 6, u = p & 63;
      int e = c * kChunk + er;
      if (e >= E) e = 0;
      const int64_t ev = ent_s[e];
      const bool pool = ev < 0;
      const int64_t row = pool ? (-ev - 1) : ev;
      if constexpr (KV == CSA2_KV_FP8_E4M3_UE8M0_32) {
        st.code[it] = *reinterpret_cast<const uint2*>((pool ? a.comp_kv : a.win_kv) + row * kDim + u * 8);
        st.sc[it] = (pool ? a.comp_scale : a.win_scale)[row * (kDim / kScaleBlock) + (u >> 2)];
      } else {  // FP4: 8 codes (4 bytes) and the E4M3 scale of their 16-value block
        st.c4[it] = *reinterpret_cast<const uint32_t*>((pool ? a.comp_kv : a.win_kv) + row * (kDim / 2) + u * 4);
        st.sc[it] = (pool ? a.comp_scale : a.win_scale)[row * (kDim / 16) + (u >> 1)];
      }
    }
  };
  auto stash = [&](int buf, const Stage& st) {
    uint8_t* base = smem + buf * kBufBytes;
#pragma unroll
    for (int it = 0; it < kPieces; ++it) {
      const int p = it * kThreads + t;
      uint4 v;
      if constexpr (KV == CSA2_KV_FP8_E4M3_UE8M0_32) {
        v = fp8x8_to_bf16x8(st.code[it], st.sc[it]);
      } else {
        v = fp4x8_e4m3_to_bf16x8(st.c4[it], st.sc[it]);
      }
      *reinterpret_cast<uint4*>(base + lds_off(p >> 6, (p & 63) * 16)) = v;
    }
  };
  Stage st0, st1;
  if (cbeg < cend) {
    fetch(cbeg, st0);
    if (cbeg + 1 < cend) fetch(cbeg + 1, st1);
    stash(0, st0);
    if (cbeg + 2 < cend) fetch(cbeg + 2, st0);
  }
  __syncthreads();
  // chunk c lives in LDS buffer (c - cbeg) & 1; after consuming it, the
  // register set holding chunk c+1 goes to the other buffer and is refilled
  // with chunk c+3
  for (int c = cbeg; c < cend; c += 2) {
    consume(smem, c);
    if (c + 1 < cend) {
      stash(1, st1);
      if (c + 3 < cend) fetch(c + 3, st1);
    }
    __syncthreads();
    if (c + 1 >= cend) break;
    consume(smem + kBufBytes, c + 1);
    if (c + 2 < cend) {
      stash(0, st0);
      if (c + 4 < cend) fetch(c + 4, st0);
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds O^T[256 dh + 16 tt + 4g + i][head] ----
  if (a.n_split == 1) {
    float M = m_run, L = l_run, f;
    if (a.sink) {
      const float s2 = a.sink[head] * kLog2e;
      const float M2 = fmaxf(M, s2);
      L = L * __builtin_amdgcn_exp2f(M - M2) + __builtin_amdgcn_exp2f(s2 - M2);
      f = __builtin_amdgcn_exp2f(M - M2) / L;
      M = M2;
    } else {
      f = (L > 0.f) ? 1.f / L : 0.f;
    }
    float* op = a.out + ((int64_t)b * kHeads + head) * kDim + dh * 256 + 4 * g;
    // de-rotation: a lane's sixteen columns of four dims meet up to eight
    // rope columns, so the query's cosines and sines are staged once per
    // workgroup in the partial-score LDS (idle since the last barrier)
    constexpr bool turn = ROPE;
    float* cs_t = &xs_s[0][0][0];
    float* sn_t = cs_t + kRopePairs;
    static_assert(sizeof(xs_s) >= 2 * kRopePairs * sizeof(float), "the rope table fits the score buffer");
    if (turn) {
      if (2 * t < a.rope.dims) {
        const float2 v = a.rope.table[(int64_t)b * kRopePairs + t];
        cs_t[t] = v.x;
        sn_t[t] = v.y;
      }
      __syncthreads();
    }
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      const f32x4 v = acc[tt] * f;
      float4 o = make_float4(v[0], v[1], v[2], v[3]);
      const int d0 = 256 * dh + 16 * tt + 4 * g;
      if (turn && d0 + 4 > a.rope.off && d0 < a.rope.off + a.rope.dims) {
        if (d0 >= a.rope.off) {
          const int i = (d0 - a.rope.off) >> 1;
          rope_turn(o.x, o.y, cs_t[i], sn_t[i]);
        }
        if (d0 + 2 < a.rope.off + a.rope.dims) {
          const int i = (d0 + 2 - a.rope.off) >> 1;
          rope_turn(o.z, o.w, cs_t[i], sn_t[i]);
        }
      }
      *reinterpret_cast<float4*>(op + tt * 16) = o;
    }
    if (a.lse && g == 0 && dh == 0)
      a.lse[(int64_t)b * kHeads + head] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
  } else {
    const int64_t slot = ((int64_t)b * a.n_split + sp) * kHeads + head;
    float* op = a.part_o + slot * kDim + dh * 256 + 4 * g;
#pragma unroll
    for (int tt = 0; tt < 16; ++tt)
      *reinterpret_cast<float4*>(op + tt * 16) = make_float4(acc[tt][0], acc[tt][1], acc[tt][2], acc[tt][3]);
    if (g == 0 && dh == 0) {
      a.part_ml[slot * 2] = m_run;
      a.part_ml[slot * 2 + 1] = l_run;
    }
  }
}

// Merge the split partials of one (query, head): log-sum-exp weights.  All
// of a thread's loads (every split's max, sum and four output values) are
// issued before the first is used, so the merge costs one memory round trip.
__global__ __launch_bounds__(128) void attend_combine(int32_t n_split, const float* __restrict__ part_o,
                                                     const float* __restrict__ part_ml,
                                                     const float* __restrict__ sink, float* __restrict__ out,
                                                     float* __restrict__ lse, RopeOut rope) {
  const int b = blockIdx.x / kHeads, h = blockIdx.x % kHeads;
  const int t = threadIdx.x;
  Rope4 rq{1.f, 0.f, 1.f, 0.f, false, false};
  if (rope.table != nullptr) rq = rope4_at(4 * t, rope.table + (int64_t)b * kRopePairs, rope);
  const int64_t slot0 = (int64_t)b * n_split * kHeads + h;
  float ms[kMaxSplit], ls[kMaxSplit];
  float4 v[kMaxSplit];
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s) {
    ms[s] = -__builtin_inff();
    ls[s] = 0.f;
    v[s] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (s < n_split) {
      const int64_t slot = slot0 + (int64_t)s * kHeads;
      ms[s] = part_ml[slot * 2];
      ls[s] = part_ml[slot * 2 + 1];
      v[s] = *reinterpret_cast<const float4*>(part_o + slot * kDim + t * 4);
    }
  }
  float M = -__builtin_inff();
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s) M = fmaxf(M, ms[s]);
  float s2 = -__builtin_inff();
  if (sink) {
    s2 = sink[h] * kLog2e;
    M = fmaxf(M, s2);
  }
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = 0.f;
  if (M != -__builtin_inff()) {
#pragma unroll
    for (int s = 0; s < kMaxSplit; ++s) {
      if (ms[s] == -__builtin_inff()) continue;  // an empty split (or none)
      const float w = __builtin_amdgcn_exp2f(ms[s] - M);
      L += w * ls[s];
      o.x += w * v[s].x, o.y += w * v[s].y, o.z += w * v[s].z, o.w += w * v[s].w;
    }
    if (sink) L += __builtin_amdgcn_exp2f(s2 - M);
  }
  const float f = (L > 0.f) ? 1.f / L : 0.f;
  *reinterpret_cast<float4*>(out + ((int64_t)b * kHeads + h) * kDim + t * 4) =
      rope4_apply(make_float4(o.x * f, o.y * f, o.z * f, o.w * f), rq);
  if (lse && t == 0) lse[(int64_t)b * kHeads + h] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
}

}  // namespace

int attend_split_for(int32_t B) {
  // aim for at least one workgroup per CU when the batch alone gives fewer
  const int n_cu = device_cu_count();
  int s = (B > 0) ? (n_cu + B - 1) / B : 1;
  return s < 1 ? 1 : (s > kMaxSplit ? kMaxSplit : s);
}

size_t attend_partial_floats(int32_t B, int n_split) {
  if (n_split <= 1) return 0;
  return (size_t)B * n_split * kHeads * (kDim + 2);
}

hipError_t launch_attend(const csa2_dims& d, int32_t B, const csa2_batch& bt, const void* q,
                         const void* win_kv, const uint8_t* win_scale, const void* comp_kv,
                         const uint8_t* comp_scale, const int32_t* topk_idx, const float* sink,
                         float* out, float* lse, int n_split, float* partial, const RopeOut& rope, hipStream_t s) {
  if (n_split > kMaxSplit) return hipErrorInvalidValue;
  if (B == 0) return hipSuccess;
  if (n_split < 1) n_split = 1;
  AttendArgs a;
  a.pos = bt.pos;
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
  a.part_o = partial;
  a.part_ml = partial ? partial + (size_t)B * n_split * kHeads * kDim : nullptr;
  a.K = d.index_topk;
  a.W = d.window;
  a.n_split = n_split;
  a.scale_log2 = d.softmax_scale * kLog2e;
  a.rope = rope;
  if (d.kv_dtype == CSA2_KV_BF16) return hipErrorInvalidValue;  // the DMA-ring kernel's
  const dim3 grid((unsigned)(B * n_split));
  const bool turn = rope.table != nullptr;
  if (d.kv_dtype == CSA2_KV_FP8_E4M3_UE8M0_32) {
    if (turn) hipLaunchKernelGGL((attend_kernel<CSA2_KV_FP8_E4M3_UE8M0_32, true>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((attend_kernel<CSA2_KV_FP8_E4M3_UE8M0_32, false>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (turn) hipLaunchKernelGGL((attend_kernel<CSA2_KV_FP4_E2M1_E4M3_16, true>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((attend_kernel<CSA2_KV_FP4_E2M1_E4M3_16, false>), grid, dim3(kThreads), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_split == 1) return e;
  return launch_attend_combine(B, n_split, a.part_o, a.part_ml, sink, out, lse, rope, s);
}

hipError_t launch_attend_combine(int32_t B, int n_split, const float* part_o, const float* part_ml, const float* sink,
                                 float* out, float* lse, const RopeOut& rope, hipStream_t s) {
  if (n_split < 1 || n_split > kMaxSplit) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attend_combine, dim3(B * kHeads), dim3(128), 0, s, n_split, part_o, part_ml, sink, out, lse, rope);
  return hipGetLastError();
}

}  // namespace csa2
