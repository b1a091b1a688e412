// Peak-rate microkernels for measurement: the instruction each tier is built
// on, issued back to back with no memory traffic, so that a tier's rate can be
// stated as a fraction of what the GPU itself sustains at its running clock
// as well as of the datasheet peak.
//
//   kind 0: V_MFMA_F64_4X4X4_4B_F64 (the exact tier's fma chains), eight
//           independent accumulators per wave; 512 flops per instruction.
//   kind 1: V_FMA_F64 on the vector ALU (the exact tier's other float64
//           work), sixteen independent chains per lane; 2 flops per lane.
//   kind 2: V_MFMA_F32_32X32X16_BF16 (the fast tier), four independent
//           accumulators per wave; 32768 flops per instruction.
//
// Workgroups of 256 threads, two per compute unit (two waves per SIMD). Each
// thread writes one float64 (a sum of its accumulators) to out[global thread
// index], so that nothing is optimised away; the values carry no meaning.

#include <cstring>

#include "../../include/det_peak.h"
#include "common.hpp"

namespace detgemm {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

template <int KIND>
__global__ void __launch_bounds__(256) peak_kernel(double* __restrict__ out, int iters) {
  const int t = threadIdx.x;
  double r = 0.0;
  if constexpr (KIND == 0) {
    const double a = 1.0 + 1e-3 * (t & 7), b = 1e-6 * (1 + (t >> 3 & 7));
    double acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f64_4x4x4f64(a, b, acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) r += acc[j];
  } else if constexpr (KIND == 1) {
    const double m = 1.0 - 1e-9, ad = 1e-9 * (1 + (t & 3));
    double x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = 1.0 + j;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = __builtin_fma(x[j], m, ad);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) r += x[j];
  } else {
    v8bf a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = static_cast<__bf16>(1.0f + 0.125f * ((t + e) & 3));
      b[e] = static_cast<__bf16>(1e-6f);
    }
    v16f acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) r += static_cast<double>(acc[j][e]);
  }
  out[static_cast<int64_t>(blockIdx.x) * 256 + t] = r;
}

}  // namespace

hipError_t launch_peak(int kind, int num_cu, int iters, double* out, double* flops, hipStream_t stream) {
  const int blocks = num_cu * 2;
  const double waves = 4.0 * blocks;
  switch (kind) {
    case 0:
      *flops = waves * iters * 8.0 * 512.0;
      hipLaunchKernelGGL(peak_kernel<0>, dim3(blocks), dim3(256), 0, stream, out, iters);
      break;
    case 1:
      *flops = waves * iters * 16.0 * 64.0 * 2.0;
      hipLaunchKernelGGL(peak_kernel<1>, dim3(blocks), dim3(256), 0, stream, out, iters);
      break;
    case 2:
      *flops = waves * iters * 4.0 * 32768.0;
      hipLaunchKernelGGL(peak_kernel<2>, dim3(blocks), dim3(256), 0, stream, out, iters);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace detgemm

extern "C" int det_peak_run(int kind, int iters, double* out, int64_t out_len, double* flops, hipStream_t stream) {
  if (kind < 0 || kind > 2 || iters < 1 || out == nullptr || flops == nullptr) return -1;
  int dev = -1;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return -4;
  }
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return -4;
  const int cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1;
  if (out_len < static_cast<int64_t>(cus) * 2 * 256) return -1;
  if (detgemm::launch_peak(kind, cus, iters, out, flops, stream) != hipSuccess) {
    (void)hipGetLastError();
    return -5;
  }
  return 0;
}
