// csa2_decode_static: the decode step for callers that cannot allocate device
// memory (work captured into a HIP graph, serving loops that forbid
// allocation).  Its scratch (index scores and split partials, what
// csa2_decode takes from the caller's workspace) is a file-scope device array
// of CSA2_STATIC_SCRATCH_BYTES that every GPU the library runs on holds until
// the process ends.
//
// In host code the array's name is only a host-side stand-in, not a device
// address: the address a kernel needs comes from hipGetSymbolAddress, taken
// once per device with that device current (each GPU holds its own copy at its
// own address) and kept here per device.  Nothing reads scratch before it is
// written in the same call (scores are written before the top-K reads them,
// partials before the merge), so no call clears it.  Calls that overlap on one
// GPU (several streams, several threads) share the array and race.
#include <mutex>

#include "csa2_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[CSA2_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once known

}  // namespace

extern "C" csa2_status csa2_decode_static(const csa2_dims* dims, int32_t B, const csa2_batch* batch, const void* q,
                                          const float* idx_q, const float* idx_w, const void* idx_k,
                                          const uint8_t* idx_k_scale, const void* win_kv, const uint8_t* win_scale,
                                          const void* comp_kv, const uint8_t* comp_scale, int32_t* topk_idx,
                                          const float* sink, float* out, float* lse, const csa2_out_rope* rope,
                                          hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return csa2::set_hip_error(e);
  if (dev < 0 || dev >= kMaxDevices) return CSA2_ERR_UNSUPPORTED;
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) return csa2::set_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
      g_scratch_ptr[dev] = p;
    }
    ptr = g_scratch_ptr[dev];
  }
  // a batch whose workspace would exceed the scratch is refused by the size
  // check of the shared implementation (CSA2_ERR_WORKSPACE) before any launch
  return csa2::decode_impl(dims, B, batch, q, idx_q, idx_w, idx_k, idx_k_scale, win_kv, win_scale, comp_kv,
                           comp_scale, topk_idx, sink, out, lse, ptr, CSA2_STATIC_SCRATCH_BYTES, rope, stream);
}
