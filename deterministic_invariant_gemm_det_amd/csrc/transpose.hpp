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

// The same copy for 2-byte elements moved as 16-byte pieces (eight elements):
// R and C multiples of 8, both buffers 16-byte aligned. A thread loads two
// row pieces of the 64 x 64 tile, and after the barrier gathers two column
// pieces from LDS (a row pitch of 132 bytes keeps the gathers on distinct
// banks) and stores each as one 16-byte write.
__global__ void __launch_bounds__(256) transpose16v_kernel(const uint16_t* __restrict__ in, int64_t R, int64_t C,
                                                           uint16_t* __restrict__ out) {
  __shared__ uint32_t t[64][33];   // row r: elements 2 i and 2 i + 1 in word i
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * 64, c0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int pr = threadIdx.x >> 3, pc = (threadIdx.x & 7) * 8;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = pr + 32 * i;
    if (r0 + r < R && c0 + pc < C) {
      const uint4 v = *reinterpret_cast<const uint4*>(in + (r0 + r) * C + c0 + pc);
      t[r][pc / 2] = v.x;
      t[r][pc / 2 + 1] = v.y;
      t[r][pc / 2 + 2] = v.z;
      t[r][pc / 2 + 3] = v.w;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int oc = pr + 32 * i;   // output row c0 + oc, elements r0 + pc .. r0 + pc + 7
    if (c0 + oc < C && r0 + pc < R) {
      uint32_t e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = (t[pc + j][oc >> 1] >> (16 * (oc & 1))) & 0xffffu;
      const uint4 w = {e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
      *reinterpret_cast<uint4*>(out + (c0 + oc) * R + r0 + pc) = w;
    }
  }
}

// Launch the copy on `stream`; R, C > 0 with at most 65535 tiles of 64 rows.
template <typename T>
inline hipError_t launch_transpose(const void* in, int64_t R, int64_t C, void* out, hipStream_t stream) {
  if (R <= 0 || C <= 0 || (R + 63) / 64 > 65535 || (C + 63) / 64 > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>((C + 63) / 64), static_cast<unsigned>((R + 63) / 64));
  const bool pieces = sizeof(T) == 2 && R % 8 == 0 && C % 8 == 0 && reinterpret_cast<uintptr_t>(in) % 16 == 0 &&
                      reinterpret_cast<uintptr_t>(out) % 16 == 0;
  if (pieces)
    hipLaunchKernelGGL(transpose16v_kernel, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(in), R, C,
                       static_cast<uint16_t*>(out));
  else
    hipLaunchKernelGGL(transpose_kernel<T>, grid, dim3(256), 0, stream, static_cast<const T*>(in), R, C,
                       static_cast<T*>(out));
  return hipGetLastError();
}

}  // namespace detgemm
