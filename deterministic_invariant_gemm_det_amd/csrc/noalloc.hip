// det_gemm_dw_noalloc: the weight gradient (det_gemm_dw_out) for callers that
// cannot allocate device memory -- code under stream capture, tight serving
// loops, harnesses that forbid hipMalloc. The workspace that the other entry
// points take from the per-stream pool comes from one statically allocated
// device array instead (64 MiB, held by every device the library runs on
// until the process ends), so the call allocates nothing.

#include "../../include/det_gemm.h"

#include <mutex>

#include "common.hpp"

namespace detgemm {
det_status_t dw_out_on_scratch(hipError_t (*scratch)(void** ptr, size_t* cap), void* dw, det_dtype_t dw_dt,
                               const void* x, const void* dy, int64_t m, int64_t k, int64_t n, det_dtype_t dt,
                               det_tier_t tier, hipStream_t stream);
}  // namespace detgemm

namespace {

static __device__ __align__(256) unsigned char scratch[DET_GEMM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];   // the array's device address on each device, once looked up

// The current device's copy of `scratch`. In host code the array's name only
// stands for the symbol; its device address differs per device and comes from
// the runtime, looked up once per device with that device current.
hipError_t scratch_of_current_device(void** ptr, size_t* cap) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  *cap = sizeof(scratch);
  return hipSuccess;
}

}  // namespace

extern "C" det_status_t det_gemm_dw_noalloc(void* dw, det_dtype_t dw_dt, const void* x, const void* dy, int64_t m,
                                            int64_t k, int64_t n, det_dtype_t dt, det_tier_t tier,
                                            hipStream_t stream) {
  return detgemm::dw_out_on_scratch(scratch_of_current_device, dw, dw_dt, x, dy, m, k, n, dt, tier, stream);
}
