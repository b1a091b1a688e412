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
//  2. ordered pass: one workgroup per 64 columns; 8 waves stage 128 tiles of
//     partials at a time in LDS while wave 0 (one lane per column) runs the
//     Neumaier pass over them in tile order, the next 128 being loaded while it
//     does. The pass state (s, c) is kept in the workspace between chunks.
// A chunk holds as many tiles as fit 64 MiB of partials (at least 128), so
// m = 8192 is one chunk.

#include <climits>

#include "common.hpp"

namespace detgemm {
namespace colsum {

constexpr int KT = 32;              // the method's tile length along the reduction
constexpr int V = 4;                // columns per lane in the tile pass
constexpr int WPB = 4;              // waves (one tile each) per workgroup in the tile pass
constexpr int COLS1 = 64 * V;       // columns per wave in the tile pass
constexpr int CB = 64;              // columns per workgroup in the ordered pass
constexpr int THREADS2 = 512;       // ordered pass: 8 waves stage, wave 0 combines
constexpr int TCH = 128;            // tiles per LDS round of the ordered pass (64 KB)
constexpr int LPT = TCH * CB / THREADS2;  // partials each thread loads per round
constexpr int64_t CHUNK_BYTES = int64_t(1) << 26;

template <int BYTES> struct VecOf;
template <> struct VecOf<8> { using type = uint2; };
template <> struct VecOf<16> { using type = uint4; };

__device__ inline void kbn_add(double& s, double& c, double p) {
  const double t = s + p;
  const double bp = t - s;
  const double ap = t - bp;
  const double e = (s - ap) + (p - bp);
  c = c + e;
  s = t;
}

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

// Neumaier pass over P[0 .. nt-1][col] in order, continuing (s, c) from state
// unless first; writes db when last, else the state.
template <typename O>
__global__ void __launch_bounds__(THREADS2) pass_kernel(const double* __restrict__ P, int64_t n, int64_t nt,
                                                        double* __restrict__ state, int first, int last,
                                                        typename O::T* __restrict__ db) {
  __shared__ double L[TCH][CB];
  const int tid = threadIdx.x, lc = tid % CB, lr = tid / CB;
  const int64_t col = static_cast<int64_t>(blockIdx.x) * CB + lc;
  const bool ok = col < n;
  double r[LPT];
  auto load = [&](int64_t base) {
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      const int64_t t = base + lr + j * (THREADS2 / CB);
      r[j] = (ok && t < nt) ? P[t * n + col] : 0.0;
    }
  };
  double s = 0.0, c = 0.0;
  if (!first && ok && tid < CB) {
    s = state[col];
    c = state[n + col];
  }
  const int64_t rounds = (nt + TCH - 1) / TCH;
  load(0);
  for (int64_t k = 0; k < rounds; ++k) {
#pragma unroll
    for (int j = 0; j < LPT; ++j) L[lr + j * (THREADS2 / CB)][lc] = r[j];
    __syncthreads();
    if (k + 1 < rounds) load((k + 1) * TCH);   // in flight during the pass below
    if (tid < CB) {
      const int cnt = static_cast<int>(nt - k * TCH < TCH ? nt - k * TCH : TCH);
      for (int t = 0; t < cnt; ++t) kbn_add(s, c, L[t][lc]);
    }
    __syncthreads();
  }
  if (tid < CB && ok) {
    if (last) {
      db[col] = round_from_f64<O>(s + c);
    } else {
      state[col] = s;
      state[n + col] = c;
    }
  }
}

template <typename E, typename O>
hipError_t launch_eo(const void* dy, int64_t m, int64_t n, void* db, int64_t chunk_tiles, hipStream_t stream) {
  using T = typename E::T;
  const int64_t tiles = (m + KT - 1) / KT;
  int64_t tck = CHUNK_BYTES / (8 * n) / TCH * TCH;
  if (tck < TCH) tck = TCH;
  if (chunk_tiles > 0) tck = chunk_tiles;
  if (tck > tiles) tck = tiles;
  const int64_t nch = (tiles + tck - 1) / tck;
  const int64_t ncb = (n + COLS1 - 1) / COLS1;
  const int64_t blocks2 = (n + CB - 1) / CB;
  if (ncb > INT_MAX || ncb * ((tck + WPB - 1) / WPB) > INT_MAX || blocks2 > INT_MAX) return hipErrorInvalidConfiguration;
  void* ws = nullptr;
  const size_t bytes = sizeof(double) * static_cast<size_t>(tck * n + (nch > 1 ? 2 * n : 0));
  hipError_t e = stream_workspace(stream, bytes, &ws);
  if (e != hipSuccess) return e;
  double* P = static_cast<double*>(ws);
  double* state = P + tck * n;
  const bool vec = n % V == 0 && reinterpret_cast<uintptr_t>(dy) % (V * sizeof(T)) == 0;
  const T* src = static_cast<const T*>(dy);
  auto* out = static_cast<typename O::T*>(db);
  for (int64_t ch = 0; ch < nch; ++ch) {
    const int64_t t0 = ch * tck, nt = tiles - t0 < tck ? tiles - t0 : tck;
    const dim3 g1(static_cast<unsigned>(ncb * ((nt + WPB - 1) / WPB))), b1(64 * WPB);
    if (vec)
      hipLaunchKernelGGL((tile_kernel<E, true>), g1, b1, 0, stream, src, m, n, t0, nt, static_cast<int>(ncb), P);
    else
      hipLaunchKernelGGL((tile_kernel<E, false>), g1, b1, 0, stream, src, m, n, t0, nt, static_cast<int>(ncb), P);
    hipLaunchKernelGGL((pass_kernel<O>), dim3(static_cast<unsigned>(blocks2)), dim3(THREADS2), 0, stream, P, n, nt,
                       state, ch == 0 ? 1 : 0, ch == nch - 1 ? 1 : 0, out);
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
