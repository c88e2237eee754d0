// Row-gather rate probe (a measurement aid for the attention's design, not
// part of the csa2 ABI): waves stream their own lists of random 1 KiB rows,
// two batches of 8 rows in flight per wave, either by LDS DMA
// (global_load_lds_dwordx4, as the bf16 attention gathers) or by loads into
// registers.  bench.py --gather-probe times it over regions of several sizes.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kNb = 8;  // rows per batch and wave

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)p;
}
__device__ __forceinline__ void dma_row16(const void* src, uint32_t lds) {
  uint32_t m0_saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(m0_saved)
               : "v"(src), "s"(lds)
               : "memory");
}
#define PROBE_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | 0x0F70)

// DMA: batch b + 1 goes out, then the wait leaves it in flight and ends batch b
template <int kWaves>
__global__ __launch_bounds__(64 * kWaves) void gather_dma(const uint4* __restrict__ rows, const int32_t* __restrict__ idx,
                                                          int per_wave, uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) uint4 lds[kWaves][2][kNb][64];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int32_t* my = idx + ((int64_t)blockIdx.x * kWaves + w) * per_wave;
  for (int i = 0; i < kNb; ++i) dma_row16(rows + (int64_t)my[i] * 64 + lane, lds_addr(&lds[w][0][i][0]));
  uint32_t acc = 0;
  for (int b = 0; b * kNb < per_wave; ++b) {
    const int nb = (b + 1) * kNb;
    if (nb < per_wave) {
      for (int i = 0; i < kNb; ++i)
        dma_row16(rows + (int64_t)my[nb + i] * 64 + lane, lds_addr(&lds[w][(b + 1) & 1][i][0]));
      PROBE_WAIT_VMCNT(kNb);
    } else {
      PROBE_WAIT_VMCNT(0);
    }
    acc ^= lds[w][b & 1][lane & (kNb - 1)][lane].x;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;  // keeps the work; never true for zeroed rows
}

// loads into registers, two batches in flight
template <int kWaves>
__global__ __launch_bounds__(64 * kWaves) void gather_reg(const uint4* __restrict__ rows, const int32_t* __restrict__ idx,
                                                          int per_wave, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63, w = (int)threadIdx.x >> 6;
  const int32_t* my = idx + ((int64_t)blockIdx.x * kWaves + w) * per_wave;
  uint4 v0[kNb], v1[kNb];
  uint32_t acc = 0;
  for (int i = 0; i < kNb; ++i) v0[i] = rows[(int64_t)my[i] * 64 + lane];
  for (int b = 0; b * kNb < per_wave; b += 2) {
    int nb = (b + 1) * kNb;
    if (nb < per_wave)
      for (int i = 0; i < kNb; ++i) v1[i] = rows[(int64_t)my[nb + i] * 64 + lane];
    for (int i = 0; i < kNb; ++i) acc ^= v0[i].x ^ v0[i].w;
    if (nb >= per_wave) break;
    nb += kNb;
    if (nb < per_wave)
      for (int i = 0; i < kNb; ++i) v0[i] = rows[(int64_t)my[nb + i] * 64 + lane];
    for (int i = 0; i < kNb; ++i) acc ^= v1[i].x ^ v1[i].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

// mode 0: LDS DMA, 1: loads into registers; waves 4 or 8 per workgroup; nwg
// workgroups; every wave gathers per_wave rows (a multiple of 8) listed in
// idx[(wg * waves + wave) * per_wave + r], each < the rows of `rows` (1 KiB
// each).  Returns a hipError_t.
extern "C" __attribute__((visibility("default"))) int csa2_probe_gather(int mode, int waves, int nwg, const void* rows,
                                                                       const int32_t* idx, int per_wave, uint32_t* sink,
                                                                       hipStream_t s) {
  if ((mode != 0 && mode != 1) || (waves != 4 && waves != 8) || nwg <= 0 || per_wave <= 0 || per_wave % kNb)
    return (int)hipErrorInvalidValue;
  const uint4* r = static_cast<const uint4*>(rows);
  if (mode == 0 && waves == 4) hipLaunchKernelGGL(gather_dma<4>, dim3(nwg), dim3(256), 0, s, r, idx, per_wave, sink);
  if (mode == 0 && waves == 8) hipLaunchKernelGGL(gather_dma<8>, dim3(nwg), dim3(512), 0, s, r, idx, per_wave, sink);
  if (mode == 1 && waves == 4) hipLaunchKernelGGL(gather_reg<4>, dim3(nwg), dim3(256), 0, s, r, idx, per_wave, sink);
  if (mode == 1 && waves == 8) hipLaunchKernelGGL(gather_reg<8>, dim3(nwg), dim3(512), 0, s, r, idx, per_wave, sink);
  return (int)hipGetLastError();
}
