// Transposed copy of a row-major matrix, for the weight-gradient paths that
// read one operand along its rows instead of down its columns. Pure data
// movement: the copy holds the same values, so the GEMM that reads it computes
// the same bits as from the original layout.
#pragma once

#include "common.hpp"

namespace detgemm {

// out[c * R + r] = in[r * C + c] for an R x C matrix of T (2- or 4-byte
// elements), through LDS in 64 x 64 tiles: rows read and columns written
// along consecutive addresses.
template <typename T>
__global__ void __launch_bounds__(256) transpose_kernel(const T* __restrict__ in, int64_t R, int64_t C,
                                                        T* __restrict__ out) {
  __shared__ T t[64][65 + (sizeof(T) == 2 ? 1 : 0)];
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * 64, c0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    if (r < R && c < C) t[i][tx] = in[r * C + c];
  }
  __syncthreads();
#pragma unroll
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < C && r < R) out[c * R + r] = t[tx][i];
  }
}

// Launch the copy on `stream`; R, C > 0 with at most 65535 tiles of 64 rows.
template <typename T>
inline hipError_t launch_transpose(const void* in, int64_t R, int64_t C, void* out, hipStream_t stream) {
  if (R <= 0 || C <= 0 || (R + 63) / 64 > 65535 || (C + 63) / 64 > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>((C + 63) / 64), static_cast<unsigned>((R + 63) / 64));
  hipLaunchKernelGGL(transpose_kernel<T>, grid, dim3(256), 0, stream, static_cast<const T*>(in), R, C,
                     static_cast<T*>(out));
  return hipGetLastError();
}

}  // namespace detgemm
