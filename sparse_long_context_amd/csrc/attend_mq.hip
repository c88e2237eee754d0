// Two-source single-softmax attention for batches of many queries with bf16
// KV (a prefill chunk, or a decode batch of a few hundred queries): one
// resident workgroup of twelve waves per CU takes (query, entry split)
// items in turn (Reading Notes of DeepSeek-V4.1-Flash, section 3f C2 Step 3;
// "DeepSeek-V4.1-Flash on WASTE", What is new, 1. CSA2): the query's 64
// heads attend, in ONE softmax, over its window rows followed by its
// selected compressed rows; every KV row is both key and value; an optional
// per-head sink logit joins only the denominator; a query with no entry
// gives zeros (PocketLLM page, "The op layer").
//
// Rows reach LDS by DMA (global_load_lds_dwordx4: lane l's 16 bytes land at
// the instruction's LDS base + 16 l), into a ring of four 32-row slots, one
// whole 1 KiB row per instruction, lane l fetching 16-byte unit l ^ f(r) of
// row r, which leaves the slot XOR-swizzled.
//
// Wave w runs on SIMD w mod 4, three waves per SIMD, and the waves split the
// work by role so that every SIMD carries the same matrix work:
//   waves 0, 1, 4, 5 (scores; two each on SIMDs 0, 1): scorer h holds Q^T of
//     heads 16 h .. +15 for all 512 dims and per chunk of 32 entries computes
//       S^T (32 entries x 16 heads) = K (32 x 512) * Q^T (512 x 16),
//     runs the online softmax of its heads in fp32 (exp2 domain, lazily
//     raised reference) and leaves P (bf16) and the heads' rescale factors
//     in LDS; while one scorer of a SIMD is in its softmax the other keeps
//     the matrix core busy;
//   waves 2, 3, 6, 7 (values; two each on SIMDs 2, 3): value wave v holds
//     O^T of dims 128 v .. +127 for all 64 heads and, one chunk behind, adds
//       O^T (128 dims x 64 heads) += V^T (128 x 32) * P^T (32 x 64),
//     V^T read transposed out of the slot (ds_read_b64_tr_b16);
//   waves 8 .. 11 (gathers, one per SIMD): build each item's entry list and
//     issue the row DMAs, 8 rows of every chunk each, two chunks ahead.
// All products are v_mfma_f32_16x16x32_bf16.  Per entry the CU reads K out of
// LDS four times and V^T once, and no partial scores cross waves.  One
// barrier per chunk: chunk c's scores and chunk c - 1's values run between
// two barriers, while chunks c + 1 and c + 2 are in flight.
//
// Workgroup i runs on XCD i mod 8 (round-robin dispatch); items are handed
// out so each XCD takes a contiguous run, which keeps the window rows that
// consecutive prefill queries share (127 of 128) in that XCD's L2.
#include <type_traits>

#include "csa2_internal.h"

namespace csa2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kWv = 12;
constexpr int kThr = 64 * kWv;
constexpr int kCh = 32;                 // entries per chunk
constexpr int kRowB = kDim * 2;         // one bf16 row
constexpr int kSlotB = kCh * kRowB;     // 32 KiB per ring slot
constexpr int kSlots = 4;               // chunk c lives in slot c % 4
constexpr int kRowsPerValuer = kCh / 4; // rows of a chunk each value wave gathers
constexpr int kPRowB = 80;              // one head's 32 probabilities (64 B), padded
constexpr int kPBufB = kHeads * kPRowB;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;  // log2 headroom before the running max is raised
constexpr int kScorer = 0, kValuer = 1, kGatherer = 2;  // wave roles

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
  RopeOut rope;      // de-rotation of unsplit outputs (splits: the merge's)
};

// 16-byte unit u of slot row r sits at unit u ^ f(r), with f(r) =
// 2 (r mod 4) + (r / 4 mod 2) + 8 ((r / 4 xor r / 8) mod 2) < 16.
//   K fragments (row r = 16-row tile row, one unit): rows 0..15 take sixteen
//     different units, rows 0..7 and 8..15 eight different units mod 8;
//   transposing reads (rows 4 g + 0..3, units 2 j and 2 j + 1, 8 bytes per
//     lane): one group of four rows takes eight different units mod 8, and
//     the groups g = 0, 1 (and 2, 3) differ in bit 3.
// So both patterns spread over all LDS banks whether a cycle serves 128 or
// 256 bytes.
__device__ __forceinline__ int swz(int r, int u) {
  return u ^ ((2 * (r & 3)) | ((r >> 2) & 1) | ((((r >> 2) ^ (r >> 3)) & 1) << 3));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)p;
}

// One 16-byte-per-lane DMA from global memory into LDS: lane l's bytes land
// at lds + 16 l.  Issued as inline assembly so that the compiler, which
// cannot tell ring slots apart, does not wait for every DMA in flight before
// each LDS read; the kernel orders the DMAs itself (a vmcnt wait, then a
// barrier, before a slot is read).
__device__ __forceinline__ void dma_row16(const void* src, uint32_t lds) {
  uint32_t m0_saved;  // the compiler treats m0 as reserved: keep its value
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "v"(src), "s"(lds)
      : "memory");
}

// s_waitcnt with only the vector-memory count constrained (expcnt and lgkmcnt
// at their maxima): vmcnt in bits 3:0 and 15:14.
#define CSA2_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | 0x0F70)

// ROPE: unsplit outputs leave de-rotated (a separate instantiation, so the
// plain kernel carries none of its code or registers)
template <bool ROPE>
__global__ __launch_bounds__(kThr) void attend_mq_kernel(MqArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kSlots * kSlotB];
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[2][kPBufB];  // P of chunk c in pbuf[c % 2]
  __shared__ float alpha_s[2][kHeads];  // rescale factor of each head, valid where flag_s is set
  __shared__ __attribute__((aligned(16))) uint32_t flag_s[2][4];  // [chunk % 2][head tile]: the tile's references moved
  __shared__ float fin_s[kHeads];       // output factor of each head
  __shared__ int64_t ent_s[kMaxEntries];  // >= 0: window row; < 0: -(pool row) - 1
  __shared__ int32_t item_e_s[2];       // entry count of the item, by item parity
  __shared__ float rope_s[2][kMaxRopeDims / 2];  // cos, sin of the rope pairs of the output leaving next

  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // wave-uniform role
  // A workgroup's waves go to the SIMDs in turn (wave w to SIMD w % 4), so
  // every SIMD holds one score wave, one value wave and one gather wave: the
  // same matrix work on each, and a score wave's softmax runs beside the
  // value wave's products (two score waves on one SIMD reach their products,
  // and their softmax, together)
  const int role = wv >= 8 ? kGatherer : (wv < 4 ? kScorer : kValuer);
  const int hq = wv & 3;  // scorer: head tile; value wave: dim quarter; gatherer: row group

  // The workgroups stay resident and take (query, split) items in turn: the
  // items form contiguous runs per XCD (workgroup i runs on XCD i % 8), and
  // the M workgroups of an XCD take every M-th item of its run, so each
  // XCD's CUs work on neighbouring queries at any time.
  const int n_items = a.B * a.n_split;
  const int nwg = (int)gridDim.x;
  const int xcd = (int)blockIdx.x & 7;
  const int m_xcd = (nwg - xcd + 7) >> 3;
  const int run_len = n_items / 8 + (xcd < n_items % 8 ? 1 : 0);
  const int run0 = xcd * (n_items / 8) + (xcd < n_items % 8 ? xcd : n_items % 8);
  const int k_first = (int)blockIdx.x >> 3;
  // One copy of the item loop per role (the role is a template constant in
  // each), so no role's registers stay live through another role's code;
  // the copies pass the same barriers: per item three while the previous
  // item's output leaves, one after the first rows have landed, one per
  // chunk, one at the end.
  auto run = [&](auto role_c) __attribute__((always_inline)) {
  constexpr int R = decltype(role_c)::value;
  constexpr bool scorer = R == kScorer, gatherer = R == kGatherer, valuer = R == kValuer;
  // ---- entry lists (gather waves): an item's metadata and selection list
  // are loaded one item ahead into the gather waves' registers (lane l holds
  // list entries 64 r + l), and each gather wave compacts the list into
  // ent_s itself (the four write the same values), so a list needs no
  // barrier of its own and the value waves' output stores of the previous
  // item drain while the first rows of the next are on their way ----
  struct Pf {
    int32_t wl, md, plen;
    int64_t w0, p0;
    float2 cs;  // (cos, sin) of the lane's rope pair (ROPE)
    int32_t idx[8];
  };
  auto prefetch = [&](int item_, int lane_) __attribute__((always_inline)) -> Pf {
    const int bb = item_ / a.n_split;
    Pf p;
    p.wl = a.win_kv ? a.win_len[bb] : 0;
    p.w0 = a.win_row0[bb];
    p.md = a.mode[bb];
    p.plen = a.pool_len[bb];
    p.p0 = a.pool_row0[bb];
    p.cs = make_float2(1.f, 0.f);
    if constexpr (ROPE)
      if (a.n_split == 1 && 2 * lane_ < a.rope.dims) p.cs = a.rope.table[(int64_t)bb * kRopePairs + lane_];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int k = 64 * r + lane_;
      p.idx[r] = (a.topk != nullptr && k < a.K) ? a.topk[(int64_t)bb * a.K + k] : -1;
    }
    return p;
  };
  Pf pf = {};
  if constexpr (gatherer)
    if (k_first < run_len) pf = prefetch(run0 + k_first, (int)threadIdx.x & 63);
  // scorers: Q^T fragments of head 16 h + l16, dims 32 s + 8 g .. +7, loaded
  // from global memory one item ahead (after the last scores of the item
  // before), so they arrive while that item's output leaves
  bf16x8 qf[16];
  auto load_q = [&](int item_) __attribute__((always_inline)) {
    int lane_ = (int)threadIdx.x & 63;
    asm volatile("" : "+v"(lane_));
    const uint16_t* qp = a.q + ((int64_t)(item_ / a.n_split) * kHeads + 16 * hq + (lane_ & 15)) * kDim + 8 * (lane_ >> 4);
#pragma unroll
    for (int s = 0; s < 16; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qp + 32 * s);
  };
  // the sink logit of the scorer lane's head (log2 units), read once, so that
  // no global load of finish() waits behind the next item's Q loads
  float sink_l2 = 0.f;
  if constexpr (scorer) {
    if (a.sink) sink_l2 = a.sink[16 * hq + ((int)threadIdx.x & 15)] * kLog2e;
    if (k_first < run_len) load_q(run0 + k_first);
  }
  // value waves: O^T tiles [dim tile][head tile]; lane holds
  // O^T[128 v + 16 dt + 4 g + k][16 ht + l16]; the output of item
  // (prev_b, prev_sp) waits in them until the next item starts
  f32x4 acc[8][4];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) acc[dt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
  int prev_b = -1, prev_sp = 0;
  // The output of item (prev_b, prev_sp) leaves in two rounds through ring
  // slots 2 and 3 (free between the end of an item and the first barrier of
  // the next): round r stages heads 32 r .. +31 as fp32 rows [32][512] (16-
  // byte unit u of row h at u ^ (h % 16), so neither the writes nor the
  // reads conflict), then value wave v stores rows 8 v .. +7 of it, each
  // instruction 1 KiB at consecutive addresses (non-temporal: nothing here
  // reads the output again).  Stored straight from the
  // accumulator layout, each instruction would cover sixteen 64-byte pieces
  // 2 KiB apart, which drain several times slower and hold up the next
  // item's loads behind them.  The lane index is re-derived opaquely, so no
  // output address stays live through the loops.
  auto stage_out = [&](auto r_c) __attribute__((always_inline)) {
    constexpr int r = decltype(r_c)::value;
    int lane_ = (int)threadIdx.x & 63;
    asm volatile("" : "+v"(lane_));
    const int g_ = lane_ >> 4, l16_ = lane_ & 15;
    uint8_t* st = ring + 2 * kSlotB;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int ht = 2 * r + t;
      const float f = fin_s[16 * ht + l16_];
      uint8_t* row = st + (16 * t + l16_) * (kDim * 4);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int u = 32 * hq + 4 * dt + g_;  // dims 128 v + 16 dt + 4 g ..
        *reinterpret_cast<f32x4*>(row + ((u ^ l16_) << 4)) = acc[dt][ht] * f;
        acc[dt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  auto store_out = [&](auto r_c, int b_, int sp_) __attribute__((always_inline)) {
    constexpr int r = decltype(r_c)::value;
    int lane_ = (int)threadIdx.x & 63;
    asm volatile("" : "+v"(lane_));
    float* obase = (a.n_split > 1 ? a.part_o + ((int64_t)b_ * a.n_split + sp_) * kHeads * kDim
                                  : a.out + (int64_t)b_ * kHeads * kDim) +
                   (32 * r + 8 * hq) * kDim + 4 * lane_;
    const uint8_t* st = ring + 2 * kSlotB + 8 * hq * (kDim * 4);
    // A finished output turns its rope pairs back.  The lane's two columns of
    // four dims lie 256 apart and the rope dims span at most 128, so at most
    // one column (half rh) meets them; a gather wave left the pairs'
    // cosines and sines in rope_s, and the column's two serve every row.
    // Every lane turns and then selects (no branch between the staged loads
    // and the stores, which would serialize them).
    auto rows = [&](auto turn_c) __attribute__((always_inline)) {
      constexpr bool turn = decltype(turn_c)::value;
      bool e0 = false, e1 = false, o0 = false, o1 = false;  // pair 0 / 1 turns in the even / odd half
      float c0 = 1.f, s0 = 0.f, c1 = 1.f, s1 = 0.f;
      if constexpr (turn) {
        const int lo = a.rope.off, hi = a.rope.off + a.rope.dims;
        const int rh = (4 * lane_ + 4 > lo && 4 * lane_ < hi) ? 0 : (4 * lane_ + 260 > lo && 4 * lane_ + 256 < hi) ? 1 : -1;
        const int d0 = 4 * lane_ + 256 * (rh > 0 ? 1 : 0);
        const bool t0 = rh >= 0 && d0 >= lo, t1 = rh >= 0 && d0 + 2 < hi;
        e0 = t0 && rh == 0, e1 = t1 && rh == 0, o0 = t0 && rh == 1, o1 = t1 && rh == 1;
        const int p0 = t0 ? (d0 - lo) >> 1 : 0, p1 = t1 ? (d0 + 2 - lo) >> 1 : 0;
        c0 = rope_s[0][p0], s0 = rope_s[1][p0], c1 = rope_s[0][p1], s1 = rope_s[1][p1];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int h = 8 * hq + (i >> 1);  // staged row
        const int u = 64 * (i & 1) + lane_;
        f32x4 v = *reinterpret_cast<const f32x4*>(st + (i >> 1) * (kDim * 4) + ((u ^ (h & 15)) << 4));
        if constexpr (turn) {
          const bool u0 = (i & 1) ? o0 : e0, u1 = (i & 1) ? o1 : e1;
          float x = v[0], y = v[1], z = v[2], w = v[3];
          rope_turn(x, y, c0, s0);
          rope_turn(z, w, c1, s1);
          v = f32x4{u0 ? x : v[0], u0 ? y : v[1], u1 ? z : v[2], u1 ? w : v[3]};
        }
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(obase + (i >> 1) * kDim + 256 * (i & 1)));
      }
    };
    if constexpr (ROPE) {
      if (a.n_split == 1) rows(std::true_type{});
      else rows(std::false_type{});
    } else {
      rows(std::false_type{});
    }
  };
  // three barriers in every role: stage, store, stage, store
  auto flush_out = [&]() __attribute__((always_inline)) {
    if constexpr (valuer) {
      if (prev_b >= 0) stage_out(std::integral_constant<int, 0>{});
      __syncthreads();
      if (prev_b >= 0) store_out(std::integral_constant<int, 0>{}, prev_b, prev_sp);
      __syncthreads();
      if (prev_b >= 0) stage_out(std::integral_constant<int, 1>{});
      __syncthreads();
      if (prev_b >= 0) store_out(std::integral_constant<int, 1>{}, prev_b, prev_sp);
    } else {
      __syncthreads();
      __syncthreads();
      __syncthreads();
    }
  };
  int par = 0;  // item parity (item_e_s)
#pragma clang loop unroll(disable)
  for (int k_item = k_first; k_item < run_len; k_item += m_xcd) {
  const int item = run0 + k_item;
  const int b = item / a.n_split, sp = item % a.n_split;
  // The lane index is re-derived opaquely for every item, so the per-lane
  // offsets are not hoisted out of the item loop.
  int lane = (int)threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int g = lane >> 4, l16 = lane & 15;
  // the item's entries and its chunks [c_beg, c_beg + nch) of the query's
  int E = 0, c_beg = 0, nch = 0;
  auto set_entries = [&](int E_) __attribute__((always_inline)) {
    E = __builtin_amdgcn_readfirstlane(E_);  // uniform: the loops run on scalars
    const int nch_all = (E + kCh - 1) / kCh;
    const int cps = (nch_all + a.n_split - 1) / a.n_split;
    c_beg = sp * cps;
    const int c_end = c_beg + cps < nch_all ? c_beg + cps : nch_all;
    nch = c_end > c_beg ? c_end - c_beg : 0;  // local chunk c is the query's c_beg + c
  };

  // Per-lane LDS offsets within a slot, for 16 x 16 x 32 fragments (lane (g,
  // l16) holds row l16 of a 16-row tile and 8 consecutive values of its
  // k-range):
  //   K of k-step s (dims 32 s + 8 g ..), entry tile et: row 16 et + l16,
  //     unit 4 s + g -> ko[s % 4] + 256 (s / 4) + 16 KiB et;
  //   V^T of dim tile dt (dims 128 v + 16 dt ..), rows 4 g + tj (+16), the
  //     transposing read's 8-byte piece -> vo0 + 32 (dt ^ vf) (+16 KiB), since
  //     (2 dt + b) ^ f(r) = 2 (dt ^ f(r) / 2) + (b ^ f(r) % 2).
  const int tj = (lane >> 2) & 3, tc = lane & 3;
  const int r_lo = 4 * g + tj;
  uint32_t ko[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) ko[j] = l16 * kRowB + (swz(l16, 4 * j + g) << 4);
  const int vf_full = swz(r_lo, 0);
  const int vf = vf_full >> 1;
  const uint32_t vo0 = r_lo * kRowB + 256 * hq + 16 * ((tc >> 1) ^ (vf_full & 1)) + 8 * (tc & 1);

  // ---- scorer state: the running reference (log2 units) of the lane's
  // head, the same in its four lanes l16 + 16 g; the sum is this lane's
  // share (reduced at the end) ----
  float m_run = -__builtin_inff(), l_run = 0.f;
  // maximum / sum over the four lanes of a head: swap with the lane 32 away,
  // then with the lane 16 away (gfx950 permlane swaps)
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

  // Scores and softmax of chunk c (scorers): P into pbuf[c % 2], the
  // rescale factors into alpha_s / flag_s of the same parity.  Lane (g, l16)
  // ends with head 16 hq + l16 and entries 4 g .. +3 of both entry tiles,
  // exactly its group of the head's P row (see the value waves' P^T).
  auto score = [&](int c, const bf16x8* qf) __attribute__((always_inline)) {
    const uint8_t* slot = ring + (c % kSlots) * kSlotB;
    f32x4 sa[2][2] = {};  // [entry tile][k-step parity]
    constexpr int kAhead = 8;  // K fragments in flight
    bf16x8 kf[kAhead];
    // read i: k-step i / 2, entry tile i % 2
    auto kread = [&](int i) __attribute__((always_inline)) -> bf16x8 {
      const int s = i >> 1, et = i & 1;
      return *reinterpret_cast<const bf16x8*>(slot + ko[s & 3] + 256 * (s >> 2) + 16 * kRowB * et);
    };
#pragma unroll
    for (int i = 0; i < kAhead; ++i) kf[i] = kread(i);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const bf16x8 k = kf[i % kAhead];
      if (i + kAhead < 32) kf[i % kAhead] = kread(i + kAhead);
      const int s = i >> 1, et = i & 1;
      sa[et][s & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k, qf[s], sa[et][s & 1], 0, 0, 0);
    }
    // keep kAhead fragment reads in flight ahead of the products (LDS reads:
    // mask 0x100, matrix ops: 0x008)
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
    for (int i = 0; i < 32 - kAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);

    float sv[8];  // entry 16 (i / 4) + 4 g + i % 4
#pragma unroll
    for (int i = 0; i < 8; ++i) sv[i] = (sa[i >> 2][0][i & 3] + sa[i >> 2][1][i & 3]) * a.scale_log2;
    if ((c_beg + c + 1) * kCh > E) {  // the query's last chunk: rows past E score -inf
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if ((c_beg + c) * kCh + 16 * (i >> 2) + 4 * g + (i & 3) >= E) sv[i] = -__builtin_inff();
    }
    float lm = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) lm = fmaxf(lm, sv[i]);
    // The reference of a head moves only when one of its scores exceeds it by
    // more than 2^kLazy, so probabilities stay below 2^kLazy.  Only when some
    // lane would move does the wave take the chunk maxima over each head's
    // four lanes and rescale.
    uint32_t moved = 0;
    if (__ballot(lm > m_run + kLazy)) {
      const float cmax = head_max(lm);
      float alpha = 1.f;
      if (cmax > m_run + kLazy) {  // false while both are -inf
        alpha = __builtin_amdgcn_exp2f(m_run - cmax);
        m_run = cmax;
      }
      l_run *= alpha;
      if (g == 0) alpha_s[c & 1][16 * hq + l16] = alpha;
      moved = 1;
    }
    if (lane == 0) flag_s[c & 1][hq] = moved;
    // every chunk holds at least one entry, so after the first the references
    // are finite
    bf16x8 pb;
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float pv = __builtin_amdgcn_exp2f(sv[i] - m_run);
      rs += pv;
      pb[i] = (__bf16)pv;
    }
    l_run += rs;
    *reinterpret_cast<bf16x8*>(pbuf[c & 1] + (16 * hq + l16) * kPRowB + 16 * g) = pb;
  };

  // Values of chunk c (value waves).  P^T operand of head tile ht: lane (g,
  // l16) takes head 16 ht + l16, entries 4 g .. +3 and 16 + 4 g .. +3 (entry
  // group g of the head's P row), matching the V^T rows of the transposed
  // reads.
  auto values = [&](int c) __attribute__((always_inline)) {
    const uint8_t* slot = ring + (c % kSlots) * kSlotB;
    const uint4 fl = *reinterpret_cast<const uint4*>(flag_s[c & 1]);
    if (__builtin_amdgcn_readfirstlane(fl.x | fl.y | fl.z | fl.w)) {
      const uint32_t f4[4] = {fl.x, fl.y, fl.z, fl.w};
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        const float al = f4[ht] ? alpha_s[c & 1][16 * ht + l16] : 1.f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc[dt][ht] *= al;
      }
    }
    bf16x8 pt[4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
      pt[ht] = *reinterpret_cast<const bf16x8*>(pbuf[c & 1] + (16 * ht + l16) * kPRowB + 16 * g);
    // re-derived opaquely per chunk so the eight tile offsets are not kept
    // in registers through the loop (the accumulators need them)
    uint32_t vbase = vo0;
    int vfx = vf;
    asm volatile("" : "+v"(vbase), "+v"(vfx));
    auto vread = [&](int dt, s16x4& lo, s16x4& hi) __attribute__((always_inline)) {
      const uint8_t* p = slot + vbase + 32 * (dt ^ vfx);
      lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((__attribute__((address_space(3))) uint8_t*)(p)));
      hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)((__attribute__((address_space(3))) uint8_t*)(p + 16 * kRowB)));
    };
    s16x4 vl[2], vh[2];
    vread(0, vl[0], vh[0]);
    vread(1, vl[1], vh[1]);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int u = dt % 2;
      const s16x8 v8 = {vl[u][0], vl[u][1], vl[u][2], vl[u][3], vh[u][0], vh[u][1], vh[u][2], vh[u][3]};
      if (dt + 2 < 8) vread(dt + 2, vl[u], vh[u]);
#pragma unroll
      for (int ht = 0; ht < 4; ++ht)
        acc[dt][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v8), pt[ht], acc[dt][ht], 0, 0, 0);
    }
    // P^T and two V^T tiles ahead, then each tile's four products followed
    // by the reads of the tile two ahead
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int dt = 0; dt < 6; ++dt) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  };

  // ---- gather of chunk c into its slot (value waves): this wave's 8 rows,
  // one DMA each; rows past the last entry repeat entry 0 (their probability
  // is 0).  Lane i < 8 looks up the entry of row i a chunk ahead
  // (entry_for); the DMAs then take each row from that lane ----
  auto entry_for = [&](int c) __attribute__((always_inline)) -> int64_t {
    int e = (c_beg + c) * kCh + kRowsPerValuer * hq + (lane & (kRowsPerValuer - 1));
    if (e >= E) e = 0;
    return ent_s[e];
  };
  auto gather = [&](int c, int64_t evl) __attribute__((always_inline)) {
    uint8_t* slot = ring + (c % kSlots) * kSlotB;
    const uint32_t lo = (uint32_t)evl, hi = (uint32_t)((uint64_t)evl >> 32);
#pragma unroll
    for (int i = 0; i < kRowsPerValuer; ++i) {
      const int r = kRowsPerValuer * hq + i;
      const int64_t ev = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, i) << 32) |
                                   (uint32_t)__builtin_amdgcn_readlane((int)lo, i));
      const uint8_t* src = (ev < 0) ? a.comp_kv + (-ev - 1) * kRowB : a.win_kv + ev * kRowB;
      dma_row16(src + (swz(r, lane) << 4), lds_addr(slot + r * kRowB));
    }
  };

  // scorer: the factor that turns a head's sum into its output, and its
  // lse (or, for entry splits, the partial max and sum)
  auto finish = [&]() __attribute__((always_inline)) {
    const float lsum = head_sum(l_run);
    if (g != 0) return;
    const int head = 16 * hq + l16;
    if (a.n_split > 1) {  // unnormalised partials, merged by attend_combine
      const int64_t pslot = ((int64_t)b * a.n_split + sp) * kHeads + head;
      a.part_ml[pslot * 2] = m_run;
      a.part_ml[pslot * 2 + 1] = lsum;
      fin_s[head] = 1.f;
      return;
    }
    float M = m_run, L = lsum, f;
    if (a.sink) {
      const float s2 = sink_l2;
      const float M2 = fmaxf(M, s2);
      L = L * __builtin_amdgcn_exp2f(M - M2) + __builtin_amdgcn_exp2f(s2 - M2);
      f = __builtin_amdgcn_exp2f(M - M2) / L;
      M = M2;
    } else {
      f = (L > 0.f) ? 1.f / L : 0.f;
    }
    fin_s[head] = f;
    if (a.lse) a.lse[(int64_t)b * kHeads + head] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
  };

  if constexpr (gatherer) {
    // ---- this item's list, then its first two chunks ----
    const Pf cur = pf;
    int wl = cur.wl;
    wl = wl < 0 ? 0 : (wl > a.W ? a.W : wl);
    for (int e = lane; e < wl; e += 64) ent_s[e] = cur.w0 + e;
    int nsel = 0;
    if (cur.md != CSA2_MODE_WINDOW && a.topk != nullptr && a.comp_kv != nullptr) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const bool ok = (cur.idx[r] >= 0) & (cur.idx[r] < cur.plen);
        const uint64_t m = __ballot(ok);
        if (ok) ent_s[wl + nsel + __popcll(m & ((1ull << lane) - 1ull))] = -(cur.p0 + cur.idx[r]) - 1;
        nsel += __popcll(m);
      }
    }
    set_entries(wl + nsel);
    if (hq == 0 && lane == 0) item_e_s[par] = E;
    // the next item's list loads go out before this item's first rows, so
    // the wait for those covers them
    if (k_item + m_xcd < run_len) pf = prefetch(item + m_xcd, lane);
    int64_t ev_next = 0;
    if (nch > 0) gather(0, entry_for(0));
    if (nch > 1) gather(1, entry_for(1));
    if (nch > 2) ev_next = entry_for(2);
    flush_out();
    if (nch > 1) CSA2_WAIT_VMCNT(kRowsPerValuer);
    else CSA2_WAIT_VMCNT(0);
    __syncthreads();
    // The cosines and sines of this item's rope pairs (loaded with its
    // list), for its output, which leaves in the next item's first rounds:
    // the previous item's output was read from rope_s before the barrier
    // just passed.
    if (ROPE && a.n_split == 1 && hq == 0 && 2 * lane < a.rope.dims) {
      rope_s[0][lane] = cur.cs.x;
      rope_s[1][lane] = cur.cs.y;
    }
#pragma clang loop unroll(disable)
    for (int c = 0; c < nch; ++c) {
      if (c + 2 < nch) {
        gather(c + 2, ev_next);
        if (c + 3 < nch) ev_next = entry_for(c + 3);
        CSA2_WAIT_VMCNT(kRowsPerValuer);
      } else {
        CSA2_WAIT_VMCNT(0);
      }
      __syncthreads();
    }
  } else if constexpr (scorer) {
    flush_out();
    __syncthreads();
    set_entries(item_e_s[par]);
#pragma clang loop unroll(disable)
    for (int c = 0; c < nch; ++c) {
      score(c, qf);
      __syncthreads();
    }
    if (k_item + m_xcd < run_len) load_q(item + m_xcd);
    finish();
  } else {
    // the previous item's output (its factors are in fin_s since the last
    // barrier) leaves while the first rows of this one are gathered
    flush_out();
    __syncthreads();
    set_entries(item_e_s[par]);
#pragma clang loop unroll(disable)
    for (int c = 0; c < nch; ++c) {
      if (c > 0) values(c - 1);
      __syncthreads();
    }
    if (nch > 0) values(nch - 1);
    prev_b = b;
    prev_sp = sp;
  }
  __syncthreads();
  par ^= 1;
  }  // items
  flush_out();  // the last item's output
  };
  // the gather waves' DMAs go out ahead of the other waves' work on their
  // SIMD (a wave's issue priority, not a stream's)
  if (role == kScorer) {
    run(std::integral_constant<int, kScorer>{});
  } else if (role == kGatherer) {
    __builtin_amdgcn_s_setprio(3);
    run(std::integral_constant<int, kGatherer>{});
  } else {
    run(std::integral_constant<int, kValuer>{});
  }
}

}  // namespace

hipError_t launch_attend_mq(const csa2_dims& d, int32_t B, const csa2_batch& bt, const void* q,
                            const void* win_kv, const void* comp_kv, const int32_t* topk_idx, const float* sink,
                            float* out, float* lse, int n_split, float* partial, const RopeOut& rope,
                            hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (n_split > kMaxSplit) return hipErrorInvalidValue;
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
  a.rope = rope;
  // one resident workgroup per CU (its LDS rules out a second), each taking
  // items in turn
  int dev = 0, n_cu = 0;
  hipError_t e0 = hipGetDevice(&dev);
  if (e0 == hipSuccess) e0 = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e0 != hipSuccess) return e0;
  const int64_t n_items = (int64_t)B * n_split;
  const int grid = (int)(n_items < n_cu ? n_items : (n_cu > 0 ? n_cu : 1));
  if (rope.table != nullptr)
    hipLaunchKernelGGL(attend_mq_kernel<true>, dim3((unsigned)grid), dim3(kThr), 0, s, a);
  else
    hipLaunchKernelGGL(attend_mq_kernel<false>, dim3((unsigned)grid), dim3(kThr), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_split == 1) return e;
  return launch_attend_combine(B, n_split, a.part_o, a.part_ml, sink, out, lse, rope, s);
}

}  // namespace csa2
