// LayerNorm over the last dimension with float64 statistics (Carbon README,
// alia-carbon 0.2.0, "How It Works", the LayerNorm row: mean and variance in
// float64 instead of a parallel reduction whose order depends on the threads).
// Every row sum is the matmul's exact-tier sum -- 32-element tiles, an
// ascending float64 chain per tile from +0, Neumaier across tiles in order:
//   mean = sum(x) / H;  d_j = x_j - mean;  var = sum(d_j * d_j) / H  (biased);
//   rstd = 1 / sqrt(var + eps);
//   y_j  = RNE((d_j * rstd) * gamma_j + beta_j)   (float64 steps, no fusion;
//          an absent gamma or beta skips its step).
// Backward, xhat_j = d_j * rstd (d_j from the stored mean), g_j = dy_j * gamma_j:
//   a = sum(g) / H;  b = sum(g_j * xhat_j) / H;
//   dx_j = RNE(rstd * ((g_j - a) - xhat_j * b));
//   dgamma_j = sum_i dy_ij * xhat_ij,  dbeta_j = sum_i dy_ij  over rows i, in
//   32-row tiles with Neumaier across them (the column sums of colsum.hpp).
// Every float64 operation is IEEE-rounded (division and square root included),
// so the results are the same bits on any device that follows the order.
//
// Forward with whole tiles and aligned operands (fwd_staged_kernel): an
// eight-wave workgroup copies up to 64 rows through LDS in 16-byte pieces,
// one thread per tile, and one lane per row runs that row's Neumaier passes.
// Other row kernels (at least four waves per SIMD, at most 128 registers,
// except the backward with more than one tile per lane): a row belongs to
// G = min(T, 64) lanes of one wave (T = tiles per row); lane g owns tiles
// g, g + G, ... and keeps their values in registers (up to TPL tiles, else it
// reads them again from memory). Each pass writes the lane's tile partials to
// LDS; one lane per row runs the Neumaier pass over them in tile order and
// shares the result through LDS. 64 / G rows share a wave (two rows of 24
// tiles for H = 768).

#include <type_traits>

#include "colsum.hpp"

namespace detgemm {
namespace ln {

constexpr int KT = 32;

// Row geometry for H = h: T tiles, G lanes per row, RW rows per wave, NW waves
// per workgroup, TPL tiles kept in registers per lane (0: re-read).
struct Geom {
  int T, G, RW, NW, TPL;
};

inline Geom geom(int64_t h) {
  Geom g;
  g.T = static_cast<int>((h + KT - 1) / KT);
  g.G = g.T < 64 ? g.T : 64;
  g.RW = 64 / g.G;
  const int per_lane = (g.T + g.G - 1) / g.G;
  g.TPL = per_lane <= 1 ? 1 : per_lane <= 2 ? 2 : 0;
  g.NW = 1;   // rows never span waves, so a one-wave workgroup needs no cross-wave barrier
  return g;
}

// The 32 (or fewer, in the last tile) values of tile t of one row, upcast
// exactly to float. VEC: the row start and every 16 bytes are aligned.
template <typename E, bool VEC>
__device__ inline void load_tile(const typename E::T* __restrict__ row, int h, int t, float (&v)[KT]) {
  using T = typename E::T;
  const int c0 = t * KT;
  if constexpr (VEC) {
    constexpr int PER = 16 / sizeof(T);
#pragma unroll
    for (int q = 0; q < KT / PER; ++q) {
      if (c0 + q * PER < h) {
        const uint4 w = *reinterpret_cast<const uint4*>(row + c0 + q * PER);
        T x[PER];
        __builtin_memcpy(x, &w, 16);
#pragma unroll
        for (int e = 0; e < PER; ++e) v[q * PER + e] = E::to_f32(x[e]);
      } else {
#pragma unroll
        for (int e = 0; e < PER; ++e) v[q * PER + e] = 0.0f;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < KT; ++e) v[e] = c0 + e < h ? E::to_f32(row[c0 + e]) : 0.0f;
  }
}

template <typename E, bool VEC>
__device__ inline void store_tile(typename E::T* __restrict__ row, int h, int t, const double (&r)[KT]) {
  using T = typename E::T;
  const int c0 = t * KT;
  if constexpr (VEC) {
    constexpr int PER = 16 / sizeof(T);
#pragma unroll
    for (int q = 0; q < KT / PER; ++q) {
      if (c0 + q * PER < h) {
        T x[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) x[e] = round_from_f64<E>(r[q * PER + e]);
        uint4 w;
        __builtin_memcpy(&w, x, 16);
        *reinterpret_cast<uint4*>(row + c0 + q * PER) = w;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < KT; ++e)
      if (c0 + e < h) row[c0 + e] = round_from_f64<E>(r[e]);
  }
}

// Elements c0 .. c0 + 7 of a row (c0 a multiple of 8), upcast exactly to
// float; elements past h read as 0. VEC: as load_tile (h is a multiple of the
// elements per 16 bytes, so every 16-byte piece lies wholly inside or outside).
template <typename E, bool VEC>
__device__ inline void load8(const typename E::T* __restrict__ row, int h, int c0, float (&v)[8]) {
  using T = typename E::T;
  if constexpr (VEC) {
    constexpr int PER = 16 / sizeof(T);
#pragma unroll
    for (int q = 0; q < 8 / PER; ++q) {
      if (c0 + q * PER < h) {
        const uint4 w = *reinterpret_cast<const uint4*>(row + c0 + q * PER);
        T x[PER];
        __builtin_memcpy(x, &w, 16);
#pragma unroll
        for (int e = 0; e < PER; ++e) v[q * PER + e] = E::to_f32(x[e]);
      } else {
#pragma unroll
        for (int e = 0; e < PER; ++e) v[q * PER + e] = 0.0f;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = c0 + e < h ? E::to_f32(row[c0 + e]) : 0.0f;
  }
}

// Elements c0 .. c0 + 7 of a row, each rounded once; nothing is written past h.
template <typename E, bool VEC>
__device__ inline void store8(typename E::T* __restrict__ row, int h, int c0, const double (&r)[8]) {
  using T = typename E::T;
  if constexpr (VEC) {
    constexpr int PER = 16 / sizeof(T);
#pragma unroll
    for (int q = 0; q < 8 / PER; ++q) {
      if (c0 + q * PER < h) {
        T x[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) x[e] = round_from_f64<E>(r[q * PER + e]);
        uint4 w;
        __builtin_memcpy(&w, x, 16);
        *reinterpret_cast<uint4*>(row + c0 + q * PER) = w;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (c0 + e < h) row[c0 + e] = round_from_f64<E>(r[e]);
  }
}

// Neumaier pass over P[0 .. T-1] in order (one lane).
// The partials are read eight at a time ahead of the dependent updates.
__device__ inline double ordered_sum(const double* P, int T) {
  double s = 0.0, c = 0.0;
  int t = 0;
  for (; t + 8 <= T; t += 8) {
    double v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = P[t + j];
#pragma unroll
    for (int j = 0; j < 8; ++j) colsum::kbn_add(s, c, v[j]);
  }
  for (; t < T; ++t) colsum::kbn_add(s, c, P[t]);
  return s + c;
}

// A lane's tiles g, g + G, ... (nk of them): kept in registers (TPL > 0; the
// loops over them are unrolled so that every register index is static) or read
// again on each visit (TPL == 0). VT: the register type of the kept values
// (float64 converts them once; float halves the registers).
template <typename E, bool VEC, int TPL, typename VT = float>
struct Tiles {
  VT v[TPL > 0 ? TPL : 1][KT];
  const typename E::T* row;
  int h, g, G, nk;
  __device__ void init(const typename E::T* r, int hh, int gg, int GG, int T) {
    row = r;
    h = hh;
    g = gg;
    G = GG;
    nk = (T - g + G - 1) / G;
    if constexpr (TPL > 0) {
#pragma unroll
      for (int k = 0; k < TPL; ++k)
        if (k < nk) {
          float tmp[KT];
          load_tile<E, VEC>(row, h, g + k * G, tmp);
#pragma unroll
          for (int e = 0; e < KT; ++e) v[k][e] = static_cast<VT>(tmp[e]);
        }
    }
  }
  // f(t, values) for each of the lane's tiles in ascending order
  template <typename F>
  __device__ void each(F&& f) {
    if constexpr (TPL > 0) {
#pragma unroll
      for (int k = 0; k < TPL; ++k)
        if (k < nk) f(g + k * G, v[k]);
    } else {
      float tmp[KT];
      for (int k = 0; k < nk; ++k) {
        load_tile<E, VEC>(row, h, g + k * G, tmp);
        f(g + k * G, tmp);
      }
    }
  }
};

// Two rows' worth of tiles visited together (x and dy of the backward).
template <typename E, bool VEC, int TPL, typename F>
__device__ inline void each2(Tiles<E, VEC, TPL, float>& a, Tiles<E, VEC, TPL, float>& b, F&& f) {
  if constexpr (TPL > 0) {
#pragma unroll
    for (int k = 0; k < TPL; ++k)
      if (k < a.nk) f(a.g + k * a.G, a.v[k], b.v[k]);
  } else {
    float ta[KT], tb[KT];
    for (int k = 0; k < a.nk; ++k) {
      load_tile<E, VEC>(a.row, a.h, a.g + k * a.G, ta);
      load_tile<E, VEC>(b.row, b.h, b.g + k * b.G, tb);
      f(a.g + k * a.G, ta, tb);
    }
  }
}

template <typename E, int TPL, bool VEC>
__global__ void __launch_bounds__(256, 4) fwd_kernel(const typename E::T* __restrict__ x,
                                                  const typename E::T* __restrict__ gamma,
                                                  const typename E::T* __restrict__ beta, int64_t rows, int h,
                                                  Geom gm, double eps, typename E::T* __restrict__ y,
                                                  double* __restrict__ mean_out, double* __restrict__ rstd_out) {
  extern __shared__ double sm[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rg = lane / gm.G, g = lane % gm.G;
  const int slot = wave * gm.RW + rg;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (gm.NW * gm.RW) + slot;
  const bool ok = rg < gm.RW && row < rows;
  const int T = gm.T, G = gm.G;
  double* P = sm + slot * T;
  double* stat = sm + gm.NW * gm.RW * T;   // [slot] mean, [NW RW + slot] rstd
  Tiles<E, VEC, TPL, typename std::conditional<TPL == 1, double, float>::type> tl;
  if (ok) tl.init(x + row * h, h, g, G, T);

  // pass 1: tile sums of x (elements past the row's end are skipped, so a
  // short last tile is the chain over its own elements)
  if (ok) {
    tl.each([&](int t, const auto& v) {
      double p = 0.0;
#pragma unroll
      for (int e = 0; e < KT; ++e)
        if (t * KT + e < h) p = p + static_cast<double>(v[e]);
      P[t] = p;
    });
  }
  __syncthreads();
  if (ok && g == 0) stat[slot] = ordered_sum(P, T) / static_cast<double>(h);
  __syncthreads();
  const double mu = ok ? stat[slot] : 0.0;

  // pass 2: tile sums of (x - mean)^2
  if (ok) {
    tl.each([&](int t, const auto& v) {
      double p = 0.0;
#pragma unroll
      for (int e = 0; e < KT; ++e) {
        if (t * KT + e < h) {
          const double d = static_cast<double>(v[e]) - mu;
          p = __builtin_fma(d, d, p);
        }
      }
      P[t] = p;
    });
  }
  __syncthreads();
  if (ok && g == 0) {
    const double var = ordered_sum(P, T) / static_cast<double>(h);
    const double rs = 1.0 / __builtin_sqrt(var + eps);
    stat[gm.NW * gm.RW + slot] = rs;
    if (mean_out) mean_out[row] = mu;
    if (rstd_out) rstd_out[row] = rs;
  }
  __syncthreads();
  if (!ok) return;
  const double rs = stat[gm.NW * gm.RW + slot];

  // pass 3: y = (d * rstd) * gamma + beta, one rounding; eight elements at a
  // time (few live registers, so that four waves fit on a SIMD)
  tl.each([&](int t, const auto& v) {
#pragma unroll
    for (int q = 0; q < KT / 8; ++q) {
      const int c0 = t * KT + 8 * q;
      float gv[8], bv[8];
      if (gamma) load8<E, VEC>(gamma, h, c0, gv);
      if (beta) load8<E, VEC>(beta, h, c0, bv);
      double r[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        double u = (static_cast<double>(v[8 * q + e]) - mu) * rs;
        if (gamma) u = u * static_cast<double>(gv[e]);
        if (beta) u = u + static_cast<double>(bv[e]);
        r[e] = u;
      }
      store8<E, VEC>(y + row * h, h, c0, r);
    }
  });
}

// Forward for rows whose length is a multiple of the tile width, with
// 16-byte aligned operands (STAGE_WAVES waves, SRW = min(64, 64 STAGE_WAVES / T)
// rows per workgroup: 21 rows of 24 tiles for H = 768). The workgroup's rows
// are one contiguous block of SRW T tiles. The block, gamma and beta move
// between memory and LDS in 16-byte pieces, consecutive lanes on consecutive
// pieces; in LDS piece q of tile f sits in slot f PPT + (q XOR ((f / (16 / PPT))
// mod PPT)), PPT = pieces per tile, which keeps the copies and the per-tile
// reads free of bank conflicts. Thread i takes tile i (row i / T, tile i mod T)
// into float64 registers: x after pass 1, x - mean after pass 2. The outputs
// go back through the tile's own slots. Thread r < SRW runs row r's two
// Neumaier passes, so one instruction stream serves all the rows.
constexpr int STAGE_WAVES = 8;
constexpr size_t STAGE_LDS_MAX = 81920;   // two workgroups per compute unit

template <typename E>
__global__ void __launch_bounds__(64 * STAGE_WAVES) fwd_staged_kernel(
    const typename E::T* __restrict__ x, const typename E::T* __restrict__ gamma,
    const typename E::T* __restrict__ beta, int64_t rows, int h, int T, int SRW, double eps,
    typename E::T* __restrict__ y, double* __restrict__ mean_out, double* __restrict__ rstd_out) {
  using TT = typename E::T;
  constexpr int PER = 16 / sizeof(TT);   // elements per piece
  constexpr int PPT = KT / PER;          // pieces per tile
  constexpr int TPG = 16 / PPT;          // tiles per 256 bytes (all 64 banks)
  constexpr int NTH = 64 * STAGE_WAVES;
  extern __shared__ uint4 smem[];
  uint4* X = smem;                                       // SRW T tiles of x, then of y
  uint4* G = X + SRW * T * PPT;                          // T tiles of gamma
  uint4* B = G + T * PPT;                                // T tiles of beta
  double* P = reinterpret_cast<double*>(B + T * PPT);    // tile partials
  double* stat = P + NTH;                                // [r] mean, [64 + r] rstd
  const auto slot = [](int f, int q) { return f * PPT + (q ^ ((f / TPG) % PPT)); };
  const int tid = threadIdx.x;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * SRW;
  const int nr = rows - row0 < SRW ? static_cast<int>(rows - row0) : SRW;
  const int ntile = nr * T;

  const uint4* xs = reinterpret_cast<const uint4*>(x + row0 * h);
  for (int i = tid; i < ntile * PPT; i += NTH) X[slot(i / PPT, i % PPT)] = xs[i];
  if (gamma) {
    const uint4* gs = reinterpret_cast<const uint4*>(gamma);
    for (int i = tid; i < T * PPT; i += NTH) G[slot(i / PPT, i % PPT)] = gs[i];
  }
  if (beta) {
    const uint4* bs = reinterpret_cast<const uint4*>(beta);
    for (int i = tid; i < T * PPT; i += NTH) B[slot(i / PPT, i % PPT)] = bs[i];
  }
  __syncthreads();

  const bool own = tid < ntile;
  const int r = tid / T, t = tid - r * T;
  double v[KT];
#pragma unroll
  for (int q = 0; q < PPT; ++q) {
    TT e8[PER];
    if (own) {
      const uint4 w = X[slot(tid, q)];
      __builtin_memcpy(e8, &w, 16);
    } else {
      __builtin_memset(e8, 0, 16);
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) v[q * PER + e] = static_cast<double>(E::to_f32(e8[e]));
  }

  // pass 1: tile sums of x
  {
    double p = 0.0;
#pragma unroll
    for (int e = 0; e < KT; ++e) p = p + v[e];
    if (own) P[tid] = p;
  }
  __syncthreads();
  const bool lead = tid < nr;
  if (lead) stat[tid] = ordered_sum(P + tid * T, T) / static_cast<double>(h);
  __syncthreads();

  // pass 2: d = x - mean kept in place; tile sums of d * d
  {
    const double mu = stat[own ? r : 0];
    double p = 0.0;
#pragma unroll
    for (int e = 0; e < KT; ++e) {
      const double d = v[e] - mu;
      v[e] = d;
      p = __builtin_fma(d, d, p);
    }
    if (own) P[tid] = p;
  }
  __syncthreads();
  if (lead) {
    const double var = ordered_sum(P + tid * T, T) / static_cast<double>(h);
    const double rs = 1.0 / __builtin_sqrt(var + eps);
    stat[64 + tid] = rs;
    if (mean_out) mean_out[row0 + tid] = stat[tid];
    if (rstd_out) rstd_out[row0 + tid] = rs;
  }
  __syncthreads();

  // pass 3: y = (d * rstd) * gamma + beta, one rounding, into the tile's own slots
  if (own) {
    const double rs = stat[64 + r];
#pragma unroll
    for (int q = 0; q < PPT; ++q) {
      TT gv[PER], bv[PER], out[PER];
      if (gamma) { const uint4 w = G[slot(t, q)]; __builtin_memcpy(gv, &w, 16); }
      if (beta) { const uint4 w = B[slot(t, q)]; __builtin_memcpy(bv, &w, 16); }
      double u[PER];
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        u[e] = v[q * PER + e] * rs;
        if (gamma) u[e] = u[e] * static_cast<double>(E::to_f32(gv[e]));
        if (beta) u[e] = u[e] + static_cast<double>(E::to_f32(bv[e]));
      }
      round_group<E>(u, out);
      uint4 w;
      __builtin_memcpy(&w, out, 16);
      X[slot(tid, q)] = w;
    }
  }
  __syncthreads();
  uint4* ys = reinterpret_cast<uint4*>(y + row0 * h);
  for (int i = tid; i < ntile * PPT; i += NTH) ys[i] = X[slot(i / PPT, i % PPT)];
}

// Backward dx for rows of whole tiles with 16-byte aligned operands, laid out
// as the staged forward: a workgroup of BWD_WAVES waves copies its rows of x
// and dy and all of gamma through LDS in 16-byte pieces; thread i keeps
// g = dy gamma and xhat of tile i in float64 registers across the two
// passes, and its dx goes back through the tile's slots of x.
#ifndef LN_BWD_WAVES
#define LN_BWD_WAVES 4
#endif
constexpr int BWD_WAVES = LN_BWD_WAVES;

template <typename E>
__global__ void __launch_bounds__(64 * BWD_WAVES) bwd_staged_kernel(
    const typename E::T* __restrict__ dy, const typename E::T* __restrict__ x, const double* __restrict__ mean,
    const double* __restrict__ rstd, const typename E::T* __restrict__ gamma, int64_t rows, int h, int T, int SRW,
    typename E::T* __restrict__ dx) {
  using TT = typename E::T;
  constexpr int PER = 16 / sizeof(TT);
  constexpr int PPT = KT / PER;
  constexpr int TPG = 16 / PPT;
  constexpr int NTH = 64 * BWD_WAVES;
  extern __shared__ uint4 smem[];
  uint4* X = smem;                                       // SRW T tiles of x, then of dx
  uint4* D = X + SRW * T * PPT;                          // SRW T tiles of dy
  uint4* G = D + SRW * T * PPT;                          // T tiles of gamma
  double* Pa = reinterpret_cast<double*>(G + T * PPT);   // tile partials of g and of g xhat
  double* Pb = Pa + NTH;
  double* stat = Pb + NTH;                               // [r] a, [64 + r] b
  const auto slot = [](int f, int q) { return f * PPT + (q ^ ((f / TPG) % PPT)); };
  const int tid = threadIdx.x;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * SRW;
  const int nr = rows - row0 < SRW ? static_cast<int>(rows - row0) : SRW;
  const int ntile = nr * T;

  const uint4* xs = reinterpret_cast<const uint4*>(x + row0 * h);
  const uint4* ds = reinterpret_cast<const uint4*>(dy + row0 * h);
  for (int i = tid; i < ntile * PPT; i += NTH) {
    X[slot(i / PPT, i % PPT)] = xs[i];
    D[slot(i / PPT, i % PPT)] = ds[i];
  }
  if (gamma) {
    const uint4* gs = reinterpret_cast<const uint4*>(gamma);
    for (int i = tid; i < T * PPT; i += NTH) G[slot(i / PPT, i % PPT)] = gs[i];
  }
  const bool own = tid < ntile;
  const int r = tid / T, t = tid - r * T;
  const double mu = own ? mean[row0 + r] : 0.0, rs = own ? rstd[row0 + r] : 0.0;
  __syncthreads();

  double gv[KT], xh[KT];
#pragma unroll
  for (int q = 0; q < PPT; ++q) {
    TT ex[PER], ed[PER], eg[PER];
    if (own) {
      const uint4 wx = X[slot(tid, q)], wd = D[slot(tid, q)];
      __builtin_memcpy(ex, &wx, 16);
      __builtin_memcpy(ed, &wd, 16);
    } else {
      __builtin_memset(ex, 0, 16);
      __builtin_memset(ed, 0, 16);
    }
    if (gamma) { const uint4 wg = G[slot(t, q)]; __builtin_memcpy(eg, &wg, 16); }
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const double d = static_cast<double>(E::to_f32(ed[e]));
      gv[q * PER + e] = gamma ? d * static_cast<double>(E::to_f32(eg[e])) : d;
      xh[q * PER + e] = (static_cast<double>(E::to_f32(ex[e])) - mu) * rs;
    }
  }

  // tile sums of g and of g * xhat
  {
    double pa = 0.0, pb = 0.0;
#pragma unroll
    for (int e = 0; e < KT; ++e) {
      pa = pa + gv[e];
      pb = __builtin_fma(gv[e], xh[e], pb);
    }
    if (own) {
      Pa[tid] = pa;
      Pb[tid] = pb;
    }
  }
  __syncthreads();
  if (tid < nr) {
    stat[tid] = ordered_sum(Pa + tid * T, T) / static_cast<double>(h);
    stat[64 + tid] = ordered_sum(Pb + tid * T, T) / static_cast<double>(h);
  }
  __syncthreads();

  // dx = rstd ((g - a) - xhat b), one rounding, into the tile's slots of x
  if (own) {
    const double a = stat[r], b = stat[64 + r];
#pragma unroll
    for (int q = 0; q < PPT; ++q) {
      double u[PER];
      TT out[PER];
#pragma unroll
      for (int e = 0; e < PER; ++e) u[e] = rs * ((gv[q * PER + e] - a) - xh[q * PER + e] * b);
      round_group<E>(u, out);
      uint4 w;
      __builtin_memcpy(&w, out, 16);
      X[slot(tid, q)] = w;
    }
  }
  __syncthreads();
  uint4* os = reinterpret_cast<uint4*>(dx + row0 * h);
  for (int i = tid; i < ntile * PPT; i += NTH) os[i] = X[slot(i / PPT, i % PPT)];
}

template <typename E, int TPL, bool VEC>
__global__ void __launch_bounds__(256, TPL == 1 ? 4 : 2) bwd_dx_kernel(const typename E::T* __restrict__ dy,
                                                     const typename E::T* __restrict__ x,
                                                     const double* __restrict__ mean, const double* __restrict__ rstd,
                                                     const typename E::T* __restrict__ gamma, int64_t rows, int h,
                                                     Geom gm, typename E::T* __restrict__ dx) {
  extern __shared__ double sm[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rg = lane / gm.G, g = lane % gm.G;
  const int slot = wave * gm.RW + rg;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (gm.NW * gm.RW) + slot;
  const bool ok = rg < gm.RW && row < rows;
  const int T = gm.T, G = gm.G, S = gm.NW * gm.RW;
  double* Pa = sm + slot * T;
  double* Pb = sm + (S + slot) * T;
  double* stat = sm + 2 * S * T;   // [slot] a, [S + slot] b
  Tiles<E, VEC, TPL> tx, tg;
  double mu = 0.0, rs = 0.0;
  if (ok) {
    tx.init(x + row * h, h, g, G, T);
    tg.init(dy + row * h, h, g, G, T);
    mu = mean[row];
    rs = rstd[row];
  }
  if (ok) {
    each2(tx, tg, [&](int t, const float(&vx)[KT], const float(&vg)[KT]) {
      float gm_[KT];
      if (gamma) load_tile<E, VEC>(gamma, h, t, gm_);
      double pa = 0.0, pb = 0.0;
#pragma unroll
      for (int e = 0; e < KT; ++e) {
        const int c = t * KT + e;
        if (c < h) {
          const double gv = gamma ? static_cast<double>(vg[e]) * static_cast<double>(gm_[e]) : static_cast<double>(vg[e]);
          const double xh = (static_cast<double>(vx[e]) - mu) * rs;
          pa = pa + gv;
          pb = __builtin_fma(gv, xh, pb);
        }
      }
      Pa[t] = pa;
      Pb[t] = pb;
    });
  }
  __syncthreads();
  if (ok && g == 0) {
    stat[slot] = ordered_sum(Pa, T) / static_cast<double>(h);
    stat[S + slot] = ordered_sum(Pb, T) / static_cast<double>(h);
  }
  __syncthreads();
  if (!ok) return;
  const double a = stat[slot], b = stat[S + slot];
  each2(tx, tg, [&](int t, const float(&vx)[KT], const float(&vg)[KT]) {
#pragma unroll
    for (int q = 0; q < KT / 8; ++q) {   // eight elements at a time (few live registers)
      const int c0 = t * KT + 8 * q;
      float gm_[8];
      if (gamma) load8<E, VEC>(gamma, h, c0, gm_);
      double r[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double gv = gamma ? static_cast<double>(vg[8 * q + e]) * static_cast<double>(gm_[e])
                                : static_cast<double>(vg[8 * q + e]);
        const double xh = (static_cast<double>(vx[8 * q + e]) - mu) * rs;
        r[e] = rs * ((gv - a) - xh * b);
      }
      store8<E, VEC>(dx + row * h, h, c0, r);
    }
  });
}

// Column tile partials for dgamma and dbeta: one wave per (row tile, 64 * 4
// columns); each lane chains over the tile's rows for 4 adjacent columns. VEC:
// h % 4 == 0 and both bases aligned to 4 elements (one 8- or 16-byte load per
// row and operand).
constexpr int CV = 4;
constexpr int CWPB = 4;

template <int BYTES> struct VecOf;
template <> struct VecOf<8> { using type = uint2; };
template <> struct VecOf<16> { using type = uint4; };

template <typename E, bool VEC>
__global__ void __launch_bounds__(64 * CWPB) param_tile_kernel(const typename E::T* __restrict__ dy,
                                                               const typename E::T* __restrict__ x,
                                                               const double* __restrict__ mean,
                                                               const double* __restrict__ rstd, int64_t rows,
                                                               int64_t h, int64_t t0, int64_t nt, int ncb,
                                                               double* __restrict__ Pg, double* __restrict__ Pb) {
  using T = typename E::T;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int cb = static_cast<int>(blockIdx.x % static_cast<unsigned>(ncb));
  const int64_t tb = blockIdx.x / static_cast<unsigned>(ncb);
  const int64_t tl = tb * CWPB + w;
  const int64_t c0 = static_cast<int64_t>(cb) * 64 * CV + lane * CV;
  if (tl >= nt || c0 >= h) return;   // no barrier in this kernel
  const int64_t r0 = (t0 + tl) * KT;
  const int cnt = static_cast<int>(rows - r0 < KT ? rows - r0 : KT);
  double pg[CV], pb[CV];
#pragma unroll
  for (int v = 0; v < CV; ++v) pg[v] = pb[v] = 0.0;
  auto step = [&](int i) {
    const int64_t r = r0 + i;
    const double mu = mean[r], rs = rstd[r];
    T dv[CV], xv[CV];
    if constexpr (VEC) {
      using Vec = typename VecOf<CV * sizeof(T)>::type;
      const Vec qd = *reinterpret_cast<const Vec*>(dy + r * h + c0);
      const Vec qx = *reinterpret_cast<const Vec*>(x + r * h + c0);
      __builtin_memcpy(dv, &qd, sizeof(qd));
      __builtin_memcpy(xv, &qx, sizeof(qx));
    } else {
#pragma unroll
      for (int v = 0; v < CV; ++v) {
        const int64_t c = c0 + v < h ? c0 + v : h - 1;   // clamped reads are never used
        dv[v] = dy[r * h + c];
        xv[v] = x[r * h + c];
      }
    }
#pragma unroll
    for (int v = 0; v < CV; ++v) {
      if (VEC || c0 + v < h) {
        const double d = E::up(dv[v]);
        const double xh = (E::up(xv[v]) - mu) * rs;
        pg[v] = __builtin_fma(d, xh, pg[v]);
        pb[v] = pb[v] + d;
      }
    }
  };
  if (cnt == KT) {
#pragma unroll 8
    for (int i = 0; i < KT; ++i) step(i);
  } else {
    for (int i = 0; i < cnt; ++i) step(i);
  }
#pragma unroll
  for (int v = 0; v < CV; ++v)
    if (VEC || c0 + v < h) {
      Pg[tl * h + c0 + v] = pg[v];
      Pb[tl * h + c0 + v] = pb[v];
    }
}

template <typename E>
hipError_t launch_fwd_e(const void* x, const void* gamma, const void* beta, int64_t rows, int64_t h, double eps,
                        void* y, double* mean, double* rstd, hipStream_t stream) {
  using T = typename E::T;
  const Geom gm = geom(h);
  {
    // the staged kernel: whole tiles, 16-byte aligned operands, and its LDS within STAGE_LDS_MAX
    const int srw = 64 * STAGE_WAVES / gm.T < 64 ? 64 * STAGE_WAVES / gm.T : 64;
    const size_t lds = static_cast<size_t>(srw + 2) * h * sizeof(T) + sizeof(double) * (64 * STAGE_WAVES + 128);
    const bool aligned = reinterpret_cast<uintptr_t>(x) % 16 == 0 && reinterpret_cast<uintptr_t>(y) % 16 == 0 &&
                         reinterpret_cast<uintptr_t>(gamma) % 16 == 0 && reinterpret_cast<uintptr_t>(beta) % 16 == 0;
    if (h % KT == 0 && aligned && srw >= 1 && lds <= STAGE_LDS_MAX) {
      const int64_t blocks = (rows + srw - 1) / srw;
      if (blocks > INT_MAX) return hipErrorInvalidConfiguration;
      hipLaunchKernelGGL((fwd_staged_kernel<E>), dim3(static_cast<unsigned>(blocks)), dim3(64 * STAGE_WAVES), lds,
                         stream, static_cast<const T*>(x), static_cast<const T*>(gamma), static_cast<const T*>(beta),
                         rows, static_cast<int>(h), gm.T, srw, eps, static_cast<T*>(y), mean, rstd);
      return hipGetLastError();
    }
  }
  const int64_t per_wg = gm.NW * gm.RW;
  const int64_t blocks = (rows + per_wg - 1) / per_wg;
  if (blocks > INT_MAX) return hipErrorInvalidConfiguration;
  const size_t lds = sizeof(double) * static_cast<size_t>(per_wg * gm.T + 2 * per_wg);
  const bool vec = h % (16 / sizeof(T)) == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(y) % 16 == 0 && reinterpret_cast<uintptr_t>(gamma) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(beta) % 16 == 0;
  const dim3 grid(static_cast<unsigned>(blocks)), block(64 * gm.NW);
  auto xs = static_cast<const T*>(x), gs = static_cast<const T*>(gamma), bs = static_cast<const T*>(beta);
  auto ys = static_cast<T*>(y);
  const int hi = static_cast<int>(h);
#define LN_FWD(TPL, VEC) \
  hipLaunchKernelGGL((fwd_kernel<E, TPL, VEC>), grid, block, lds, stream, xs, gs, bs, rows, hi, gm, eps, ys, mean, rstd)
  if (vec) {
    switch (gm.TPL) {
      case 1: LN_FWD(1, true); break;
      case 2: LN_FWD(2, true); break;
      default: LN_FWD(0, true); break;
    }
  } else {
    switch (gm.TPL) {
      case 1: LN_FWD(1, false); break;
      case 2: LN_FWD(2, false); break;
      default: LN_FWD(0, false); break;
    }
  }
#undef LN_FWD
  return hipGetLastError();
}

template <typename E, typename O>
hipError_t launch_params(const void* dy, const void* x, const double* mean, const double* rstd, int64_t rows,
                         int64_t h, void* dgamma, void* dbeta, hipStream_t stream) {
  using T = typename E::T;
  const colsum::Chunks ck = colsum::plan_chunks(rows, h, 0);
  const int64_t ncb = (h + 64 * CV - 1) / (64 * CV);
  if (ncb > INT_MAX || ncb * ((ck.tck + CWPB - 1) / CWPB) > INT_MAX) return hipErrorInvalidConfiguration;
  void* ws = nullptr;
  hipError_t e = stream_workspace(stream, ck.bytes(h, 2), &ws);
  if (e != hipSuccess) return e;
  double* Pg = ck.partials(ws, h, 0);
  double* Pb = ck.partials(ws, h, 1);
  double* Sg = ck.state(ws, h, 2, 0);
  double* Sb = ck.state(ws, h, 2, 1);
  const bool vec = h % CV == 0 && reinterpret_cast<uintptr_t>(dy) % (CV * sizeof(T)) == 0 &&
                   reinterpret_cast<uintptr_t>(x) % (CV * sizeof(T)) == 0;
  for (int64_t ch = 0; ch < ck.nch; ++ch) {
    const int64_t t0 = ch * ck.tck, nt = ck.tiles - t0 < ck.tck ? ck.tiles - t0 : ck.tck;
    const dim3 g1(static_cast<unsigned>(ncb * ((nt + CWPB - 1) / CWPB))), b1(64 * CWPB);
    if (vec)
      hipLaunchKernelGGL((param_tile_kernel<E, true>), g1, b1, 0, stream, static_cast<const T*>(dy),
                         static_cast<const T*>(x), mean, rstd, rows, h, t0, nt, static_cast<int>(ncb), Pg, Pb);
    else
      hipLaunchKernelGGL((param_tile_kernel<E, false>), g1, b1, 0, stream, static_cast<const T*>(dy),
                         static_cast<const T*>(x), mean, rstd, rows, h, t0, nt, static_cast<int>(ncb), Pg, Pb);
    const bool first = ch == 0, last = ch == ck.nch - 1;
    // dgamma and dbeta in one launch (their ordered passes run side by side)
    auto* og = static_cast<typename O::T*>(dgamma);
    auto* ob = static_cast<typename O::T*>(dbeta);
    if (og)
      colsum::launch_pass<O>(Pg, Sg, og, ob ? Pb : nullptr, ob ? Sb : nullptr, ob, h, nt, first, last, stream);
    else
      colsum::launch_pass<O>(Pb, Sb, ob, nullptr, nullptr, nullptr, h, nt, first, last, stream);
  }
  return hipGetLastError();
}

template <typename E>
hipError_t launch_bwd_e(bool pf32, const void* dy, const void* x, const double* mean, const double* rstd,
                        const void* gamma, int64_t rows, int64_t h, void* dx, void* dgamma, void* dbeta,
                        hipStream_t stream) {
  using T = typename E::T;
  bool dx_done = false;
  if (dx) {
    // the staged kernel: whole tiles, 16-byte aligned operands, and its LDS within STAGE_LDS_MAX
    const int Tt = static_cast<int>((h + KT - 1) / KT);
    const int srw = 64 * BWD_WAVES / Tt < 64 ? 64 * BWD_WAVES / Tt : 64;
    const size_t lds = static_cast<size_t>(2 * srw + 1) * h * sizeof(T) + sizeof(double) * (2 * 64 * BWD_WAVES + 128);
    const bool aligned = reinterpret_cast<uintptr_t>(x) % 16 == 0 && reinterpret_cast<uintptr_t>(dy) % 16 == 0 &&
                         reinterpret_cast<uintptr_t>(dx) % 16 == 0 && reinterpret_cast<uintptr_t>(gamma) % 16 == 0;
    if (h % KT == 0 && aligned && srw >= 1 && lds <= STAGE_LDS_MAX) {
      const int64_t blocks = (rows + srw - 1) / srw;
      if (blocks > INT_MAX) return hipErrorInvalidConfiguration;
      hipLaunchKernelGGL((bwd_staged_kernel<E>), dim3(static_cast<unsigned>(blocks)), dim3(64 * BWD_WAVES), lds, stream,
                         static_cast<const T*>(dy), static_cast<const T*>(x), mean, rstd, static_cast<const T*>(gamma),
                         rows, static_cast<int>(h), Tt, srw, static_cast<T*>(dx));
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      dx_done = true;
    }
  }
  if (dx && !dx_done) {
    const Geom gm = geom(h);
    const int64_t per_wg = gm.NW * gm.RW;
    const int64_t blocks = (rows + per_wg - 1) / per_wg;
    if (blocks > INT_MAX) return hipErrorInvalidConfiguration;
    const size_t lds = sizeof(double) * static_cast<size_t>(2 * per_wg * gm.T + 2 * per_wg);
    const bool vec = h % (16 / sizeof(T)) == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(dy) % 16 == 0 && reinterpret_cast<uintptr_t>(dx) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(gamma) % 16 == 0;
    const dim3 grid(static_cast<unsigned>(blocks)), block(64 * gm.NW);
    auto dys = static_cast<const T*>(dy), xs = static_cast<const T*>(x), gs = static_cast<const T*>(gamma);
    auto dxs = static_cast<T*>(dx);
    const int hi = static_cast<int>(h);
#define LN_BWD(TPL, VEC)                                                                                       \
  hipLaunchKernelGGL((bwd_dx_kernel<E, TPL, VEC>), grid, block, lds, stream, dys, xs, mean, rstd, gs, rows, hi, \
                     gm, dxs)
    if (vec) {
      switch (gm.TPL) {
        case 1: LN_BWD(1, true); break;
        case 2: LN_BWD(2, true); break;
        default: LN_BWD(0, true); break;
      }
    } else {
      switch (gm.TPL) {
        case 1: LN_BWD(1, false); break;
        case 2: LN_BWD(2, false); break;
        default: LN_BWD(0, false); break;
      }
    }
#undef LN_BWD
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!dgamma && !dbeta) return hipSuccess;
  return pf32 ? launch_params<E, F32>(dy, x, mean, rstd, rows, h, dgamma, dbeta, stream)
              : launch_params<E, E>(dy, x, mean, rstd, rows, h, dgamma, dbeta, stream);
}

}  // namespace ln

hipError_t launch_layernorm_fwd(Dt dt, const void* x, const void* gamma, const void* beta, int64_t rows, int64_t h,
                                double eps, void* y, double* mean, double* rstd, hipStream_t stream) {
  switch (dt) {
    case DT_F32: return ln::launch_fwd_e<F32>(x, gamma, beta, rows, h, eps, y, mean, rstd, stream);
    case DT_BF16: return ln::launch_fwd_e<BF16>(x, gamma, beta, rows, h, eps, y, mean, rstd, stream);
    case DT_F16: return ln::launch_fwd_e<F16>(x, gamma, beta, rows, h, eps, y, mean, rstd, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_layernorm_bwd(Dt dt, bool param_f32, const void* dy, const void* x, const double* mean,
                                const double* rstd, const void* gamma, int64_t rows, int64_t h, void* dx,
                                void* dgamma, void* dbeta, hipStream_t stream) {
  switch (dt) {
    case DT_F32: return ln::launch_bwd_e<F32>(false, dy, x, mean, rstd, gamma, rows, h, dx, dgamma, dbeta, stream);
    case DT_BF16:
      return ln::launch_bwd_e<BF16>(param_f32, dy, x, mean, rstd, gamma, rows, h, dx, dgamma, dbeta, stream);
    case DT_F16:
      return ln::launch_bwd_e<F16>(param_f32, dy, x, mean, rstd, gamma, rows, h, dx, dgamma, dbeta, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace detgemm
