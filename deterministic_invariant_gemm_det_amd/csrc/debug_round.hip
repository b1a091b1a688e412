// Test hooks: the tiers' output roundings on values chosen by the caller, on
// the device, with the very functions the epilogues call -- round_from_f32
// (fast tier: f32 accumulator to the output type), round_from_f64 (exact
// and correctly rounded tiers, LayerNorm: round to odd at f32, then the
// hardware's round to nearest even) and round_group (the LayerNorm forward's
// eight values per lane, with the wave's choice of path). The final rounding is one step of the
// computation (sgemm-bi 0.1.2 PyPI page, "Determinism contracts": the RNE
// downcast); these hooks let it be compared with the oracle over every f32
// input and over chosen float64 inputs.

#include "common.hpp"

namespace detgemm {
namespace {

constexpr int THREADS = 256;
constexpr int64_t MAX_BLOCKS = 65536;

template <typename E>
__global__ void __launch_bounds__(THREADS) round_f32_kernel(typename E::T* __restrict__ out, uint32_t first,
                                                            int64_t count) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * THREADS;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * THREADS + threadIdx.x; i < count; i += stride)
    out[i] = round_from_f32<E>(__uint_as_float(first + static_cast<uint32_t>(i)));
}

template <typename E>
__global__ void __launch_bounds__(THREADS) round_f64_kernel(typename E::T* __restrict__ out,
                                                            const double* __restrict__ in, int64_t count) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * THREADS;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * THREADS + threadIdx.x; i < count; i += stride)
    out[i] = round_from_f64<E>(in[i]);
}

// Eight consecutive values per thread through round_group; values past the
// end are padding (zero) and are not stored.
template <typename E>
__global__ void __launch_bounds__(THREADS) round_f64_grouped_kernel(typename E::T* __restrict__ out,
                                                                    const double* __restrict__ in, int64_t count) {
  const int64_t groups = (count + 7) / 8;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * THREADS;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * THREADS + threadIdx.x; g < groups; g += stride) {
    double u[8];
    typename E::T o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) u[e] = 8 * g + e < count ? in[8 * g + e] : 0.0;
    round_group<E>(u, o);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (8 * g + e < count) out[8 * g + e] = o[e];
  }
}

unsigned blocks_for(int64_t count) {
  const int64_t b = (count + THREADS - 1) / THREADS;
  return static_cast<unsigned>(b < MAX_BLOCKS ? b : MAX_BLOCKS);
}

}  // namespace

hipError_t launch_round_f32(Dt dt, void* out, uint32_t first, int64_t count, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  const dim3 grid(blocks_for(count)), block(THREADS);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(round_f32_kernel<BF16>, grid, block, 0, stream, static_cast<uint16_t*>(out), first, count);
  else if (dt == DT_F16)
    hipLaunchKernelGGL(round_f32_kernel<F16>, grid, block, 0, stream, static_cast<_Float16*>(out), first, count);
  else
    hipLaunchKernelGGL(round_f32_kernel<F32>, grid, block, 0, stream, static_cast<float*>(out), first, count);
  return hipGetLastError();
}

hipError_t launch_round_f64(Dt dt, void* out, const double* in, int64_t count, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  const dim3 grid(blocks_for(count)), block(THREADS);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(round_f64_kernel<BF16>, grid, block, 0, stream, static_cast<uint16_t*>(out), in, count);
  else if (dt == DT_F16)
    hipLaunchKernelGGL(round_f64_kernel<F16>, grid, block, 0, stream, static_cast<_Float16*>(out), in, count);
  else
    hipLaunchKernelGGL(round_f64_kernel<F32>, grid, block, 0, stream, static_cast<float*>(out), in, count);
  return hipGetLastError();
}

hipError_t launch_round_f64_grouped(Dt dt, void* out, const double* in, int64_t count, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  const dim3 grid(blocks_for((count + 7) / 8)), block(THREADS);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(round_f64_grouped_kernel<BF16>, grid, block, 0, stream, static_cast<uint16_t*>(out), in, count);
  else if (dt == DT_F16)
    hipLaunchKernelGGL(round_f64_grouped_kernel<F16>, grid, block, 0, stream, static_cast<_Float16*>(out), in, count);
  else
    hipLaunchKernelGGL(round_f64_grouped_kernel<F32>, grid, block, 0, stream, static_cast<float*>(out), in, count);
  return hipGetLastError();
}

}  // namespace detgemm
