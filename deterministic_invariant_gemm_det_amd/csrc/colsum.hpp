// Ordered column sums over row tiles: the second half of a column reduction in
// the exact tier's arithmetic (float64 tile partials already computed, one per
// 32-row tile and column, in a workspace), shared by the bias gradient and the
// LayerNorm parameter gradients.
//
// The ordered pass: one workgroup per 64 columns (and per array, when one
// launch carries two column sums); 8 waves stage 128 tiles of partials at a
// time in LDS while wave 0 (one lane per column) runs the Neumaier pass over
// them in tile order, the next 128 being loaded while it does. Long reductions are cut into chunks of whole tiles whose partials fit
// the workspace; the pass state (s, c) is kept there between chunks.
#pragma once

#include <climits>

#include "common.hpp"

namespace detgemm {
namespace colsum {

constexpr int KT = 32;              // the method's tile length along the reduction
constexpr int CB = 64;              // columns per workgroup in the ordered pass
constexpr int THREADS2 = 512;       // ordered pass: 8 waves stage, wave 0 combines
constexpr int TCH = 128;            // tiles per LDS round of the ordered pass (64 KB)
constexpr int LPT = TCH * CB / THREADS2;  // partials each thread loads per round
constexpr int64_t CHUNK_BYTES = int64_t(1) << 26;   // partials of one array per chunk

__device__ inline void kbn_add(double& s, double& c, double p) {
  const double t = s + p;
  const double bp = t - s;
  const double ap = t - bp;
  const double e = (s - ap) + (p - bp);
  c = c + e;
  s = t;
}

// Up to two column-sum arrays handled by one launch (blockIdx.y picks one):
// partials P[a], state[a], output out[a] (null: that array is skipped).
template <typename O>
struct PassArrays {
  const double* P[2];
  double* state[2];
  typename O::T* out[2];
};

// Neumaier pass over P[0 .. nt-1][col] in order, continuing (s, c) from state
// unless first; writes the output when last, else the state.
template <typename O>
__global__ void __launch_bounds__(THREADS2) pass_kernel(PassArrays<O> arr, int64_t n, int64_t nt, int first, int last) {
  __shared__ double L[TCH][CB];
  const int a = blockIdx.y;
  const double* __restrict__ P = arr.P[a];
  double* __restrict__ state = arr.state[a];
  typename O::T* __restrict__ out = arr.out[a];
  if (out == nullptr) return;   // uniform over the workgroup: no barrier is skipped by part of it
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
    if (tid < CB) {   // partials read eight at a time ahead of the dependent updates
      const int cnt = static_cast<int>(nt - k * TCH < TCH ? nt - k * TCH : TCH);
      int t = 0;
      for (; t + 8 <= cnt; t += 8) {
        double v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = L[t + j][lc];
#pragma unroll
        for (int j = 0; j < 8; ++j) kbn_add(s, c, v[j]);
      }
      for (; t < cnt; ++t) kbn_add(s, c, L[t][lc]);
    }
    __syncthreads();
  }
  if (tid < CB && ok) {
    if (last) {
      out[col] = round_from_f64<O>(s + c);
    } else {
      state[col] = s;
      state[n + col] = c;
    }
  }
}

// Chunking of `tiles` row tiles over n columns with `arrays` partial arrays:
// tck tiles per chunk (as many as fit CHUNK_BYTES per array, at least TCH,
// or chunk_tiles when > 0), nch chunks. Workspace layout: array a's partials
// at a * tck * n, then array a's state (2n values) at arrays * tck * n + 2 a n.
struct Chunks {
  int64_t tiles, tck, nch;
  size_t bytes(int64_t n, int arrays) const {
    return sizeof(double) * static_cast<size_t>(arrays) * static_cast<size_t>(tck * n + (nch > 1 ? 2 * n : 0));
  }
  double* partials(void* ws, int64_t n, int a) const { return static_cast<double*>(ws) + a * tck * n; }
  double* state(void* ws, int64_t n, int arrays, int a) const {
    return static_cast<double*>(ws) + arrays * tck * n + 2 * a * n;
  }
};

inline Chunks plan_chunks(int64_t m, int64_t n, int64_t chunk_tiles) {
  Chunks c;
  c.tiles = (m + KT - 1) / KT;
  c.tck = CHUNK_BYTES / (8 * n) / TCH * TCH;
  if (c.tck < TCH) c.tck = TCH;
  if (chunk_tiles > 0) c.tck = chunk_tiles;
  if (c.tck > c.tiles) c.tck = c.tiles;
  c.nch = (c.tiles + c.tck - 1) / c.tck;
  return c;
}

// One launch for up to two arrays (P1, state1, out1 may be null).
template <typename O>
inline void launch_pass(const double* P0, double* state0, typename O::T* out0, const double* P1, double* state1,
                        typename O::T* out1, int64_t n, int64_t nt, bool first, bool last, hipStream_t stream) {
  const int64_t blocks = (n + CB - 1) / CB;
  PassArrays<O> arr{{P0, P1}, {state0, state1}, {out0, out1}};
  hipLaunchKernelGGL((pass_kernel<O>), dim3(static_cast<unsigned>(blocks), out1 ? 2u : 1u), dim3(THREADS2), 0, stream,
                     arr, n, nt, first ? 1 : 0, last ? 1 : 0);
}

}  // namespace colsum
}  // namespace detgemm
