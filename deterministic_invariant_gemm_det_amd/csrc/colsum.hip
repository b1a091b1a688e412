// Bias gradient: db[n] = sum_i dy[i, n] (sgemm-bi 0.1.2 PyPI page, note after
// "Determinism contracts": the bias gradient is a column sum of dY, left to
// the framework there), with the exact tier's arithmetic for a reduction over
// the m rows (Carbon README, alia-carbon 0.2.0, "How It Works") -- bit for bit
// the dW of a column of ones:
//   p_t = float64 chain over rows 32t .. 32t + 31 in ascending order from +0
//         (each step adds one upcast value: fma(1, dy, p) = p + dy exactly
//         rounded once);
//   (s, c) <- Neumaier(s, c, p_t) for t ascending; db = round(s + c).
// Both tiers use this arithmetic: the op reads m x n values and does O(m n)
// additions, so it is bound by reading dY and the extra float64 work is free.
//
// Two launches per chunk of tiles:
//  1. tile pass: one wave per (tile, 256 columns); each lane runs the chains of
//     4 adjacent columns over the tile's 32 rows (8- or 16-byte row loads, so
//     a wave reads 512 or 1024 contiguous bytes per row) and writes the float64
//     partials P[t][c] to the stream's workspace. All tiles run in parallel.
//  2. the ordered Neumaier pass per column (colsum.hpp).
// A chunk holds as many tiles as fit 64 MiB of partials (at least 128), so
// m = 8192 is one chunk.

#include "colsum.hpp"

namespace detgemm {
namespace colsum {

constexpr int V = 4;                // columns per lane in the tile pass
constexpr int WPB = 4;              // waves (one tile each) per workgroup in the tile pass
constexpr int COLS1 = 64 * V;       // columns per wave in the tile pass

template <int BYTES> struct VecOf;
template <> struct VecOf<8> { using type = uint2; };
template <> struct VecOf<16> { using type = uint4; };

// P[tl][c] for tiles t0 .. t0 + nt - 1 (tl = t - t0), all columns.
// VEC: n % V == 0 and dy aligned to V elements, so each lane's V columns are one
// aligned vector load per row.
template <typename E, bool VEC>
__global__ void __launch_bounds__(64 * WPB) tile_kernel(const typename E::T* __restrict__ dy, int64_t m, int64_t n,
                                                        int64_t t0, int64_t nt, int ncb, double* __restrict__ P) {
  using T = typename E::T;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int cb = static_cast<int>(blockIdx.x % static_cast<unsigned>(ncb));
  const int64_t tb = blockIdx.x / static_cast<unsigned>(ncb);
  const int64_t tl = tb * WPB + w;
  const int64_t c0 = static_cast<int64_t>(cb) * COLS1 + lane * V;
  if (tl >= nt || c0 >= n) return;   // no barrier in this kernel
  const int64_t r0 = (t0 + tl) * KT;
  const int rows = static_cast<int>(m - r0 < KT ? m - r0 : KT);
  const T* src = dy + r0 * n + c0;
  double p[V];
#pragma unroll
  for (int v = 0; v < V; ++v) p[v] = 0.0;
  if constexpr (VEC) {
    using Vec = typename VecOf<V * sizeof(T)>::type;
    auto row = [&](int i) {
      const Vec q = *reinterpret_cast<const Vec*>(src + static_cast<int64_t>(i) * n);
      T x[V];
      __builtin_memcpy(x, &q, sizeof(q));
#pragma unroll
      for (int v = 0; v < V; ++v) p[v] = p[v] + E::up(x[v]);
    };
    if (rows == KT) {
#pragma unroll
      for (int i = 0; i < KT; ++i) row(i);
    } else {
      for (int i = 0; i < rows; ++i) row(i);
    }
    double* dst = P + tl * n + c0;
    reinterpret_cast<double2*>(dst)[0] = make_double2(p[0], p[1]);
    reinterpret_cast<double2*>(dst)[1] = make_double2(p[2], p[3]);
  } else {
    for (int i = 0; i < rows; ++i) {
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (c0 + v < n) p[v] = p[v] + E::up(src[static_cast<int64_t>(i) * n + v]);
    }
    double* dst = P + tl * n + c0;
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (c0 + v < n) dst[v] = p[v];
  }
}

template <typename E, typename O>
hipError_t launch_eo(const void* dy, int64_t m, int64_t n, void* db, int64_t chunk_tiles, hipStream_t stream) {
  using T = typename E::T;
  const Chunks ck = plan_chunks(m, n, chunk_tiles);
  const int64_t ncb = (n + COLS1 - 1) / COLS1;
  if (ncb > INT_MAX || ncb * ((ck.tck + WPB - 1) / WPB) > INT_MAX || (n + CB - 1) / CB > INT_MAX)
    return hipErrorInvalidConfiguration;
  void* ws = nullptr;
  hipError_t e = stream_workspace(stream, ck.bytes(n, 1), &ws);
  if (e != hipSuccess) return e;
  double* P = ck.partials(ws, n, 0);
  double* state = ck.state(ws, n, 1, 0);
  const bool vec = n % V == 0 && reinterpret_cast<uintptr_t>(dy) % (V * sizeof(T)) == 0;
  const T* src = static_cast<const T*>(dy);
  auto* out = static_cast<typename O::T*>(db);
  for (int64_t ch = 0; ch < ck.nch; ++ch) {
    const int64_t t0 = ch * ck.tck, nt = ck.tiles - t0 < ck.tck ? ck.tiles - t0 : ck.tck;
    const dim3 g1(static_cast<unsigned>(ncb * ((nt + WPB - 1) / WPB))), b1(64 * WPB);
    if (vec)
      hipLaunchKernelGGL((tile_kernel<E, true>), g1, b1, 0, stream, src, m, n, t0, nt, static_cast<int>(ncb), P);
    else
      hipLaunchKernelGGL((tile_kernel<E, false>), g1, b1, 0, stream, src, m, n, t0, nt, static_cast<int>(ncb), P);
    launch_pass<O>(P, state, out, nullptr, nullptr, nullptr, n, nt, ch == 0, ch == ck.nch - 1, stream);
  }
  return hipGetLastError();
}

}  // namespace colsum
hipError_t launch_db(Dt dt, bool out_f32, const void* dy, int64_t m, int64_t n, void* db, int64_t chunk_tiles,
                     hipStream_t stream) {
  switch (dt) {
    case DT_F32: return colsum::launch_eo<F32, F32>(dy, m, n, db, chunk_tiles, stream);
    case DT_BF16:
      return out_f32 ? colsum::launch_eo<BF16, F32>(dy, m, n, db, chunk_tiles, stream)
                     : colsum::launch_eo<BF16, BF16>(dy, m, n, db, chunk_tiles, stream);
    case DT_F16:
      return out_f32 ? colsum::launch_eo<F16, F32>(dy, m, n, db, chunk_tiles, stream)
                     : colsum::launch_eo<F16, F16>(dy, m, n, db, chunk_tiles, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace detgemm
