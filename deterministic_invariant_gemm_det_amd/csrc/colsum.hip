// Bias gradient: db[n] = sum_i dy[i, n] (sgemm-bi 0.1.2 PyPI page, note after
// "Determinism contracts": the bias gradient is a column sum of dY, left to
// the framework there), with the exact
// tier's arithmetic for a reduction over the m rows (Carbon README, alia-carbon
// 0.2.0, "How It Works") -- bit for bit the dW of a column of ones:
//   p_t = float64 chain over rows 32t .. 32t + 31 in ascending order from +0
//         (each step adds one upcast value: fma(1, dy, p) = p + dy exactly
//         rounded once);
//   (s, c) <- Neumaier(s, c, p_t) for t ascending; db = round(s + c).
// The op reads m x n values and does O(m n) additions, so it is bound by
// memory and the latency of the ordered pass; both tiers use this arithmetic.
//
// Workgroup: 256 threads = 8 row groups x 32 columns. The tile partials are
// independent of one another, so the row groups compute them in parallel for
// up to TC tiles at a time into LDS; then one thread per column runs the
// Neumaier pass over them in tile order, carrying (s, c) to the next chunk of
// tiles. Consecutive lanes read consecutive columns of one row.

#include "common.hpp"

namespace detgemm {
namespace colsum {

constexpr int CB = 32;            // columns per workgroup
constexpr int RG = 8;             // row groups
constexpr int THREADS = CB * RG;
constexpr int KT = 32;            // the method's tile width along the reduction
constexpr int TC = 256;           // tiles per LDS chunk (64 KB of float64 partials)

__device__ inline void kbn_add(double& s, double& c, double p) {
  const double t = s + p;
  const double bp = t - s;
  const double ap = t - bp;
  const double e = (s - ap) + (p - bp);
  c = c + e;
  s = t;
}

template <typename E, typename O>
__global__ void __launch_bounds__(THREADS) db_kernel(const typename E::T* __restrict__ dy, int64_t m, int64_t n,
                                                     typename O::T* __restrict__ db) {
  __shared__ double P[TC][CB];
  const int c = threadIdx.x % CB, rg = threadIdx.x / CB;
  const int64_t col = static_cast<int64_t>(blockIdx.x) * CB + c;
  const bool ok = col < n;
  const int64_t colc = ok ? col : n - 1;   // lanes past the last column read a valid one, never stored
  const int64_t T = (m + KT - 1) / KT;
  double s = 0.0, cc = 0.0;
  for (int64_t t0 = 0; t0 < T; t0 += TC) {
    const int nt = static_cast<int>(T - t0 < TC ? T - t0 : TC);
    for (int j = rg; j < nt; j += RG) {
      const int64_t r0 = (t0 + j) * KT;
      const typename E::T* src = dy + r0 * n + colc;
      double p = 0.0;
      if (r0 + KT <= m) {
#pragma unroll
        for (int i = 0; i < KT; ++i) p = p + E::up(src[i * n]);
      } else {
        for (int64_t i = 0; r0 + i < m; ++i) p = p + E::up(src[i * n]);   // short last tile
      }
      P[j][c] = p;
    }
    __syncthreads();
    if (rg == 0)
      for (int j = 0; j < nt; ++j) kbn_add(s, cc, P[j][c]);
    __syncthreads();
  }
  if (rg == 0 && ok) db[col] = round_from_f64<O>(s + cc);
}

template <typename E>
hipError_t launch_e(bool out_f32, const void* dy, int64_t m, int64_t n, void* db, hipStream_t stream) {
  const int64_t blocks = (n + CB - 1) / CB;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks)), block(THREADS);
  const auto* src = static_cast<const typename E::T*>(dy);
  if (out_f32)
    hipLaunchKernelGGL((db_kernel<E, F32>), grid, block, 0, stream, src, m, n, static_cast<float*>(db));
  else
    hipLaunchKernelGGL((db_kernel<E, E>), grid, block, 0, stream, src, m, n, static_cast<typename E::T*>(db));
  return hipGetLastError();
}

}  // namespace colsum

hipError_t launch_db(Dt dt, bool out_f32, const void* dy, int64_t m, int64_t n, void* db, hipStream_t stream) {
  switch (dt) {
    case DT_F32: return colsum::launch_e<F32>(false, dy, m, n, db, stream);
    case DT_BF16: return colsum::launch_e<BF16>(out_f32, dy, m, n, db, stream);
    case DT_F16: return colsum::launch_e<F16>(out_f32, dy, m, n, db, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace detgemm
