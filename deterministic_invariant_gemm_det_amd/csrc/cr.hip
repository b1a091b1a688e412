// Correctly rounded tier: every output is the exact value of its dot product
// (+ bias) rounded once to the output type (Carbon README, alia-carbon 0.2.0,
// "Roadmap", v0.2: exact summation with a superaccumulator, so that the result
// no longer depends on any order). Exactness makes the result independent of
// the reduction order, the tiling and the launch.
//
// How the exact value is reached on the matrix of the GEMM, in three launches:
//
//  1. stats: for every row r of A (the output-row operand, over the reduction)
//     the highest set bit top_r and the lowest set bit low_r of its nonzero
//     values, and for every column c of B the same; with a forward bias the
//     rows also count the value 1 and the columns their bias (the bias is the
//     product 1 * b_c at one extra reduction index). Maximum and minimum are
//     order-free, so the partial results of the workgroups meet in global
//     atomics. Non-finite values set a flag.
//
//  2. sliced tiles: a value v of row r is cut into 23-bit slices at fixed
//     positions below top_r: slice s holds the bits of v with weights
//     2^(top_r - 23 s - 22) .. 2^(top_r - 23 s), as a signed integer a_s below
//     2^23 (so v = sum_s a_s 2^(top_r - 23 s - 22), exactly). The same for the
//     columns of B. A prepass writes the first two slices of every value as
//     float32 (exact) in a K-major, zero-padded layout. For one slice pair
//     (s, t) the integer products a_s b_t are below 2^46, so the float64 matrix
//     instructions summing 128 of them stay below 2^53 and are exact in any
//     order; each such block sum is added to an int64, and the pairs are
//     combined in an int128 at their offsets 23 (s + t). A tile whose rows or
//     columns need at most two slices (span of set bits <= 46) and hold only
//     finite values is finished here: the int128 is rounded to odd at 53 bits
//     (truncate, set the last bit when anything was dropped), scaled by its
//     power of two, and rounded to the output type by the same single-rounding
//     path as the other tiers; rounding to odd first and then to a format at
//     least two bits narrower is one correct rounding (Boldo and Melquiond,
//     IEEE TC 2008).
//
// For 16-bit inputs faster forms of 2 run first (2b, 2c below): 7-bit slices
// on the int8 matrix instructions (exact int32 sums), then 8-bit slices on the
// bf16 ones (exact float32 sums over 256 reduction indices); the tiles they
// cannot take (wider spans, non-finite values) go on to 2.
//
// A null A operand stands for a column of ones (the bias gradient as the
// correctly rounded column sum of dY).
//
//  3. fallback: tiles flagged by 2 (wide spans or non-finite values) are
//     summed one output at a time in a superaccumulator: 21 int64 chunks of 32
//     bits each in LDS, covering every bit a product or bias can carry (2^-350
//     .. 2^632), each float64 product added at its bit position; carries are
//     propagated once at the end, and the integer is rounded as in 2. Sums with
//     an infinity or a NaN give the float64 sum of those terms.
//
// Both ways give the same bits for a tile (they compute the same exact value),
// so the split between them changes only the speed.

#include <climits>

#include "common.hpp"

namespace detgemm {
namespace cr {

constexpr int TILE = 64;
constexpr int KB = 32;                 // reduction indices per exact float64 block
constexpr int SLICE = 23;              // bits per slice
constexpr int NOBITS = -100000;        // "no set bit" markers of an all-zero row or column
constexpr int NOLOW = 100000;
constexpr int NCH = 21;                // superaccumulator chunks
constexpr int OFF = 352;               // bit index of 2^0 in the superaccumulator

// Sign, integer significand and the weight of its last bit of one stored value.
struct Parts {
  uint32_t sig;
  int lsb;
  bool neg, finite;
};

template <typename E> __device__ inline Parts parts(typename E::T v);
template <> __device__ inline Parts parts<F32>(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t e = (u >> 23) & 0xffu, f = u & 0x7fffffu;
  Parts p;
  p.neg = (u >> 31) != 0;
  p.finite = e != 0xffu;
  p.sig = e ? (f | 0x800000u) : f;
  p.lsb = e ? static_cast<int>(e) - 150 : -149;
  return p;
}
template <> __device__ inline Parts parts<BF16>(uint16_t v) {
  const uint32_t e = (v >> 7) & 0xffu, f = v & 0x7fu;
  Parts p;
  p.neg = (v >> 15) != 0;
  p.finite = e != 0xffu;
  p.sig = e ? (f | 0x80u) : f;
  p.lsb = e ? static_cast<int>(e) - 134 : -133;
  return p;
}
template <> __device__ inline Parts parts<F16>(_Float16 v) {
  uint16_t u;
  __builtin_memcpy(&u, &v, 2);
  const uint32_t e = (u >> 10) & 0x1fu, f = u & 0x3ffu;
  Parts p;
  p.neg = (u >> 15) != 0;
  p.finite = e != 0x1fu;
  p.sig = e ? (f | 0x400u) : f;
  p.lsb = e ? static_cast<int>(e) - 25 : -24;
  return p;
}

// highest and lowest set bit of a nonzero significand at weight 2^lsb
__device__ inline int top_bit(const Parts& p) { return p.lsb + 31 - __builtin_clz(p.sig); }
__device__ inline int low_bit(const Parts& p) { return p.lsb + __builtin_ctz(p.sig); }

// Slice s of a value whose row or column has top bit `top`: the bits with
// weights 2^(top - SLICE s - SLICE + 1) .. 2^(top - SLICE s) as a signed integer.
__device__ inline double slice(const Parts& p, int top, int s) {
  if (p.sig == 0) return 0.0;
  const int low = top - SLICE * s - (SLICE - 1);
  const int sh = p.lsb - low;
  constexpr uint64_t mask = (uint64_t(1) << SLICE) - 1;
  uint64_t part;
  if (sh >= 0)
    part = sh >= SLICE ? 0 : ((static_cast<uint64_t>(p.sig) << sh) & mask);
  else
    part = -sh >= 32 ? 0 : ((static_cast<uint64_t>(p.sig) >> (-sh)) & mask);
  const double d = static_cast<double>(part);
  return p.neg ? -d : d;
}

// 2^x as a float64, -1022 <= x <= 1023
__device__ inline double pow2(int x) { return __longlong_as_double(static_cast<long long>(x + 1023) << 52); }

// Round to odd at 53 bits of the integer z (two's complement, |z| < 2^126),
// times 2^scale. The result is a float64 from which one further rounding to a
// format of at most 51 bits is the correct rounding of z * 2^scale.
__device__ inline double round_odd53(__int128 z, int scale) {
  if (z == 0) return 0.0;
  const bool neg = z < 0;
  unsigned __int128 mag = neg ? static_cast<unsigned __int128>(-z) : static_cast<unsigned __int128>(z);
  const uint64_t hi = static_cast<uint64_t>(mag >> 64), lo = static_cast<uint64_t>(mag);
  const int n = hi ? 128 - __builtin_clzll(hi) : 64 - __builtin_clzll(lo);
  uint64_t top;
  int sh = 0;
  if (n <= 53) {
    top = lo;
  } else {
    sh = n - 53;
    top = static_cast<uint64_t>(mag >> sh);
    const unsigned __int128 rest = mag - (static_cast<unsigned __int128>(top) << sh);
    if (rest != 0) top |= 1u;
  }
  const double d = static_cast<double>(top) * pow2(scale + sh);   // exact: top < 2^53, power of two in range
  return neg ? -d : d;
}

// ---- 1. stats ---------------------------------------------------------------

// Stats of a 2D array X[outer][inner] (inner contiguous) per outer index
// (PER_OUTER: reduced over inner) or per inner index (reduced over outer).
// Each thread folds a strip and meets the others in atomics.
template <typename E, bool PER_OUTER>
__global__ void __launch_bounds__(256) stats_kernel(const typename E::T* __restrict__ X, int64_t outer, int64_t inner,
                                                    int64_t strip, int* __restrict__ top, int* __restrict__ low,
                                                    int* __restrict__ bad) {
  const int64_t nidx = PER_OUTER ? outer : inner;     // indices the stats are kept for
  const int64_t red = PER_OUTER ? inner : outer;      // length reduced over
  int t = NOBITS, lo = NOLOW, nf = 0;
  int64_t idx;
  if constexpr (PER_OUTER) {
    // a wave per outer index and strip; lanes along the contiguous dimension
    const int lane = threadIdx.x & 63;
    const int64_t w = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
    const int64_t strips = (red + strip - 1) / strip;
    idx = w / strips;
    if (idx >= nidx) return;
    const int64_t r0 = (w % strips) * strip, r1 = r0 + strip < red ? r0 + strip : red;
    for (int64_t r = r0 + lane; r < r1; r += 64) {
      const Parts p = parts<E>(X[idx * inner + r]);
      if (!p.finite) nf = 1;
      else if (p.sig) {
        t = max(t, top_bit(p));
        lo = min(lo, low_bit(p));
      }
    }
    for (int o = 32; o > 0; o >>= 1) {
      t = max(t, __shfl_xor(t, o));
      lo = min(lo, __shfl_xor(lo, o));
      nf |= __shfl_xor(nf, o);
    }
    if (lane != 0) return;
  } else {
    // a thread per inner index and strip of outer rows; lanes along the contiguous dimension
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    idx = tid % inner;
    const int64_t s = tid / inner;
    const int64_t r0 = s * strip;
    if (r0 >= red) return;
    const int64_t r1 = r0 + strip < red ? r0 + strip : red;
    for (int64_t r = r0; r < r1; ++r) {
      const Parts p = parts<E>(X[r * inner + idx]);
      if (!p.finite) nf = 1;
      else if (p.sig) {
        t = max(t, top_bit(p));
        lo = min(lo, low_bit(p));
      }
    }
  }
  if (t != NOBITS) {
    atomicMax(top + idx, t);
    atomicMin(low + idx, lo);
  }
  if (nf) atomicOr(bad + idx, 1);
}

// The per-row stats from 16-byte pieces (V = 16 / sizeof(T) values each), for
// arrays whose contiguous length, reduced length and base allow it.
template <typename E>
__device__ inline Parts parts_at(const uint4& v, int i) {
  typename E::T x;
  __builtin_memcpy(&x, reinterpret_cast<const char*>(&v) + i * sizeof(x), sizeof(x));
  return parts<E>(x);
}
template <typename E>
__device__ inline void fold(const Parts& p, int& t, int& lo, int& nf) {
  if (!p.finite) nf = 1;
  else if (p.sig) {
    t = max(t, top_bit(p));
    lo = min(lo, low_bit(p));
  }
}

// per row of X[rows][ld], over its first red values: a wave per row
template <typename E>
__global__ void __launch_bounds__(256) stats_rows_vec_kernel(const typename E::T* __restrict__ X, int64_t rows,
                                                             int64_t red, int64_t ld, int* __restrict__ top,
                                                             int* __restrict__ low, int* __restrict__ bad) {
  constexpr int V = 16 / sizeof(typename E::T);
  const int lane = threadIdx.x & 63;
  const int64_t row = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  if (row >= rows) return;
  const uint4* p = reinterpret_cast<const uint4*>(X + row * ld);
  const int64_t np = red / V;
  int t = NOBITS, lo = NOLOW, nf = 0;
  for (int64_t q = lane; q < np; q += 64) {
    const uint4 v = p[q];
#pragma unroll
    for (int i = 0; i < V; ++i) fold<E>(parts_at<E>(v, i), t, lo, nf);
  }
  for (int o = 32; o > 0; o >>= 1) {
    t = max(t, __shfl_xor(t, o));
    lo = min(lo, __shfl_xor(lo, o));
    nf |= __shfl_xor(nf, o);
  }
  if (lane != 0) return;
  if (t != NOBITS) {
    atomicMax(top + row, t);
    atomicMin(low + row, lo);
  }
  if (nf) atomicOr(bad + row, 1);
}

// per column of X[red][ld], columns 0 .. cols - 1: a workgroup per 64 16-byte
// pieces of a row (64 V columns) and strip of rows, its four waves on every
// fourth row; the waves meet in LDS and one atomic per column and workgroup
// goes out
template <typename E>
__global__ void __launch_bounds__(256) stats_cols_vec_kernel(const typename E::T* __restrict__ X, int64_t red,
                                                             int64_t cols, int64_t ld, int64_t strip,
                                                             int* __restrict__ top, int* __restrict__ low,
                                                             int* __restrict__ bad) {
  constexpr int V = 16 / sizeof(typename E::T);
  __shared__ int sh[3][4][64 * V];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t npc = cols / V, groups = (npc + 63) / 64;
  const int64_t cg = blockIdx.x % groups;
  const int64_t r0 = blockIdx.x / groups * strip, r1 = r0 + strip < red ? r0 + strip : red;
  const int64_t pc = cg * 64 + lane;
  int t[V], lo[V], nf[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    t[i] = NOBITS;
    lo[i] = NOLOW;
    nf[i] = 0;
  }
  if (pc < npc) {
#pragma unroll 4
    for (int64_t r = r0 + wave; r < r1; r += 4) {
      const uint4 v = reinterpret_cast<const uint4*>(X + r * ld)[pc];
#pragma unroll
      for (int i = 0; i < V; ++i) fold<E>(parts_at<E>(v, i), t[i], lo[i], nf[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < V; ++i) {
    sh[0][wave][lane * V + i] = t[i];
    sh[1][wave][lane * V + i] = lo[i];
    sh[2][wave][lane * V + i] = nf[i];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < 64 * V; c += 256) {
    const int64_t col = cg * 64 * V + c;
    if (col >= cols) continue;
    int tt = NOBITS, ll = NOLOW, ff = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      tt = max(tt, sh[0][w][c]);
      ll = min(ll, sh[1][w][c]);
      ff |= sh[2][w][c];
    }
    if (tt != NOBITS) {
      atomicMax(top + col, tt);
      atomicMin(low + col, ll);
    }
    if (ff) atomicOr(bad + col, 1);
  }
}

// Initial values of the stats, plus the extra values: 1 for every A row, the
// bias for every B column (when `extra` is set for that side).
template <typename E>
__global__ void __launch_bounds__(256) stats_init_kernel(int64_t rows, int64_t cols, int* __restrict__ topA,
                                                         int* __restrict__ lowA, int* __restrict__ badA,
                                                         int* __restrict__ topB, int* __restrict__ lowB,
                                                         int* __restrict__ badB,
                                                         const typename E::T* __restrict__ bias, int ones_a,
                                                         int* __restrict__ left) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < 2) left[i] = 0;
  if (i < rows) {
    topA[i] = (bias || ones_a) ? 0 : NOBITS;   // the value 1 at the bias index, or A all ones
    lowA[i] = (bias || ones_a) ? 0 : NOLOW;
    badA[i] = 0;
  }
  if (i < cols) {
    int t = NOBITS, lo = NOLOW, nf = 0;
    if (bias) {
      const Parts p = parts<E>(bias[i]);
      if (!p.finite) nf = 1;
      else if (p.sig) {
        t = top_bit(p);
        lo = low_bit(p);
      }
    }
    topB[i] = t;
    lowB[i] = lo;
    badB[i] = nf;
  }
}

__device__ inline int slices_of(int t, int lo) { return t == NOBITS ? 0 : (t - lo + SLICE) / SLICE; }

// ---- operand access ---------------------------------------------------------

// A(r, l) and B(l, c) of the GEMM, with the bias index l == red: A = 1, B = bias.
template <typename E, bool A_RC>
__device__ inline Parts a_at(const GemmArgs& g, int64_t r, int64_t l) {
  using T = typename E::T;
  const T* A = static_cast<const T*>(g.A);
  if (l == g.red || !A) {   // bias index, or A a column of ones
    Parts p;
    p.neg = false;
    p.finite = true;
    p.sig = 1;
    p.lsb = 0;
    return p;
  }
  return parts<E>(A_RC ? A[r * g.lda + l] : A[l * g.lda + r]);
}
template <typename E, bool B_RC>
__device__ inline Parts b_at(const GemmArgs& g, int64_t l, int64_t c) {
  using T = typename E::T;
  if (l == g.red) return parts<E>(static_cast<const T*>(g.bias)[c]);
  const T* B = static_cast<const T*>(g.B);
  return parts<E>(B_RC ? B[c * g.ldb + l] : B[l * g.ldb + c]);
}

struct Stats {
  const int *topA, *lowA, *badA, *topB, *lowB, *badB;
  int* flag;   // per tile: 1 when the next path must finish it
  int* left;   // tiles left by the int8 path [0] and by the bf16 path [1]
};

// ---- 2. sliced tiles ---------------------------------------------------------

// The two leading slices of every operand value, as float32 (exact: integers
// below 2^23), laid out K-major and zero-padded: S[s][l][x] for l < ktp (the
// reduction with the bias index, rounded up to 32) and x < np (rows of A or
// columns of B, rounded up to 64), so that a tile's block is one aligned,
// unconditional read. Rows or columns that need more slices are finished by
// the fallback, so two suffice here.
template <typename E, bool IS_A, bool RC>
__device__ inline void slice_prep_one(const GemmArgs& g, const int* __restrict__ top, int64_t n, int64_t np,
                                      int64_t ktp, float* __restrict__ S, int64_t i) {
  const int64_t l = i / np, x = i % np;
  float s0 = 0.0f, s1 = 0.0f;
  const int64_t kt = g.red + (g.bias ? 1 : 0);
  if (x < n && l < kt) {
    const Parts p = IS_A ? a_at<E, RC>(g, x, l) : b_at<E, RC>(g, l, x);
    if (p.finite && p.sig) {
      const int t = top[x];
      s0 = static_cast<float>(slice(p, t, 0));
      s1 = static_cast<float>(slice(p, t, 1));
    }
  }
  S[l * np + x] = s0;
  S[ktp * np + l * np + x] = s1;
}

// both operands in one grid-stride launch (A's ktp x npa elements, then B's)
template <typename E, bool A_RC, bool B_RC>
__global__ void __launch_bounds__(256) slice_prep_kernel(GemmArgs g, const int* __restrict__ topA,
                                                         const int* __restrict__ topB, int64_t npa, int64_t npb,
                                                         int64_t ktp, float* __restrict__ SA, float* __restrict__ SB,
                                                         const int* __restrict__ need) {
  if (need && *need == 0) return;   // the 16-bit paths left no tile (uniform over the grid)
  const int64_t na = ktp * npa, total = na + ktp * npb;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    if (i < na)
      slice_prep_one<E, true, A_RC>(g, topA, g.rows, npa, ktp, SA, i);
    else
      slice_prep_one<E, false, B_RC>(g, topB, g.cols, npb, ktp, SB, i - na);
  }
}

typedef double v4d __attribute__((ext_vector_type(4)));
constexpr int LSD = 80;   // LDS row stride in doubles: the four k rows a wave reads per step land in alternate bank halves
constexpr int SUBS = 4;   // 32-index stages per exact block (128 indices: 128 products below 2^46 stay below 2^53)

template <typename O>
__global__ void __launch_bounds__(256) sliced_kernel(GemmArgs g, Stats st, int tiles_c, int force_fallback,
                                                     const float* __restrict__ SA, const float* __restrict__ SB,
                                                     int64_t npa, int64_t npb, int64_t ktp, int after8) {
  __shared__ double As[KB][LSD];
  __shared__ double Bs[KB][LSD];
  __shared__ int red_s[4];
  const int tid = threadIdx.x;
  const int tile = blockIdx.x;
  if (after8 && !st.flag[tile]) return;   // finished by the 8-bit path (uniform over the workgroup)
  const int64_t r0 = static_cast<int64_t>(tile / tiles_c) * TILE, c0 = static_cast<int64_t>(tile % tiles_c) * TILE;

  // the tile's slice counts and non-finite flag
  if (tid < 4) red_s[tid] = 0;
  __syncthreads();
  {
    const int i = tid & 63;
    if (tid < 64 && r0 + i < g.rows) {
      atomicMax(&red_s[0], slices_of(st.topA[r0 + i], st.lowA[r0 + i]));
      if (st.badA[r0 + i]) atomicOr(&red_s[2], 1);
    } else if (tid >= 64 && tid < 128 && c0 + i < g.cols) {
      atomicMax(&red_s[1], slices_of(st.topB[c0 + i], st.lowB[c0 + i]));
      if (st.badB[c0 + i]) atomicOr(&red_s[2], 1);
    }
  }
  __syncthreads();
  const int LA = red_s[0], LB = red_s[1];
  const bool fallback = force_fallback || red_s[2] || LA > 2 || LB > 2;
  if (tid == 0) st.flag[tile] = fallback ? 1 : 0;
  if (fallback) return;   // uniform over the workgroup

  // A wave owns 32 x 32 outputs as 2 x 2 blocks of V_MFMA_F64_16X16X4 (accumulator e
  // of lane l: row 4e + l/16, column l%16 of its block).
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  const int lr = lane & 15, lk = lane >> 4;
  int trow[2][4], tcol[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t c = c0 + wn + 16 * i + lr;
    tcol[i] = c < g.cols ? st.topB[c] : NOBITS;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t r = r0 + wm + 16 * i + 4 * e + lk;
      trow[i][e] = r < g.rows ? st.topA[r] : NOBITS;
    }
  }
  // staging: thread copies 4 consecutive x at reduction rows lq and lq + 16 of the stage
  const int sx = 4 * (tid % 16), lq = tid / 16;

  __int128 Z[2][2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) Z[i][j][e] = 0;

  const int64_t nstages = ktp / KB;
  for (int s = 0; s < LA; ++s) {
    for (int t = 0; t < LB; ++t) {
      const float* sa = SA + s * ktp * npa + r0 + sx;
      const float* sb = SB + t * ktp * npb + c0 + sx;
      const int shift = 2 * SLICE - SLICE * (s + t);
      float4 ra[2], rb[2];
      auto load = [&](int64_t kb) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          ra[h] = *reinterpret_cast<const float4*>(sa + (kb + lq + 16 * h) * npa);
          rb[h] = *reinterpret_cast<const float4*>(sb + (kb + lq + 16 * h) * npb);
        }
      };
      int64_t I[2][2][4];
      v4d p[2][2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          p[i][j] = v4d{0.0, 0.0, 0.0, 0.0};
#pragma unroll
          for (int e = 0; e < 4; ++e) I[i][j][e] = 0;
        }
      int blocks = 0;
      load(0);
      for (int64_t st_i = 0; st_i < nstages; ++st_i) {
        __syncthreads();   // the previous stage's reads of As, Bs are done
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          double* da = &As[lq + 16 * h][sx];
          double* db = &Bs[lq + 16 * h][sx];
          da[0] = ra[h].x; da[1] = ra[h].y; da[2] = ra[h].z; da[3] = ra[h].w;
          db[0] = rb[h].x; db[1] = rb[h].y; db[2] = rb[h].z; db[3] = rb[h].w;
        }
        __syncthreads();
        if (st_i + 1 < nstages) load((st_i + 1) * KB);   // in flight during the stage below
#pragma unroll
        for (int gk = 0; gk < KB / 4; ++gk) {
          const int kr = 4 * gk + lk;
          const double a0 = As[kr][wm + lr], a1 = As[kr][wm + 16 + lr];
          const double b0 = Bs[kr][wn + lr], b1 = Bs[kr][wn + 16 + lr];
          p[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, p[0][0], 0, 0, 0);
          p[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, p[0][1], 0, 0, 0);
          p[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, p[1][0], 0, 0, 0);
          p[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, p[1][1], 0, 0, 0);
        }
        // every SUBS stages (and at the end) the block sums, integers below 2^53, go to int64
        if ((st_i + 1) % SUBS == 0 || st_i + 1 == nstages) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
              for (int e = 0; e < 4; ++e) I[i][j][e] += static_cast<int64_t>(p[i][j][e]);
              p[i][j] = v4d{0.0, 0.0, 0.0, 0.0};
            }
          if (++blocks == 1024) {   // keep the int64 below 2^63
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
              for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  Z[i][j][e] += static_cast<__int128>(I[i][j][e]) << shift;
                  I[i][j][e] = 0;
                }
            blocks = 0;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) Z[i][j][e] += static_cast<__int128>(I[i][j][e]) << shift;
    }
  }
  // Z counts units of 2^(top_r + top_c - 4 SLICE + 2): slice pair (s, t) has unit
  // 2^(top_r - SLICE (s + 1) + 1 + top_c - SLICE (t + 1) + 1) and sits SLICE (2 - s - t) bits up.
  using OT = typename O::T;
  OT* out = static_cast<OT*>(g.out);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t c = c0 + wn + 16 * j + lr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t r = r0 + wm + 16 * i + 4 * e + lk;
        if (r < g.rows && c < g.cols) {
          const double v = Z[i][j][e] == 0 ? 0.0 : round_odd53(Z[i][j][e], trow[i][e] + tcol[j] - 4 * SLICE + 2);
          out[r * g.cols + c] = round_from_f64<O>(v);
        }
      }
    }
}

// ---- 2b. 7-bit slices on the int8 matrix instructions (16-bit inputs) --------
//
// The same exact value from narrow slices on the integer matrix pipe. A value
// of row r is cut into 7-bit slices below top_r: slice j holds the bits with
// weights 2^(top_r - 7 j - 6) .. 2^(top_r - 7 j) as a signed integer of
// magnitude below 2^7 (an int8). V_MFMA_I32_16X16X64_I8 multiplies and sums
// them exactly in int32; all pairs (s, t) of one weight class q = s + t (at
// most S7MAX of them) share one accumulator, whose sums stay below
// 5 * 16384 * 127^2 < 2^31 over 16384 reduction indices, after which (and at
// the end) each class goes into the int128 at 7 (qmax - q) bits up; the int128
// is rounded as in 2. Per stage of 128 reduction indices the workgroup stages
// every slice of its 64 rows and 64 columns once (direct-to-LDS loads) and runs
// every slice pair from registers. A tile is taken here when its rows and
// columns need at most S7MAX slices (top and lowest set bit at most 34 apart)
// and all its values are finite; the others are flagged for 2c.
constexpr int S7 = 7;                // bits per slice
constexpr int S7MAX = 5;             // slices per value on this path
constexpr int NQ7 = 2 * S7MAX - 1;   // weight classes
constexpr int K7 = 128;              // reduction indices per stage (128 bytes of int8 per row)
constexpr int FL7 = 16384 / K7;      // stages per exact int32 sum

__device__ inline int slices7_of(int t, int lo) { return t == NOBITS ? 0 : (t - lo + S7) / S7; }

// Slice j of a value whose row or column has top bit `top`, as a signed integer.
__device__ inline int slice7(const Parts& p, int top, int j) {
  if (p.sig == 0) return 0;
  const int low = top - S7 * j - (S7 - 1);
  const int sh = p.lsb - low;
  uint32_t part;
  if (sh >= 0)
    part = sh >= S7 ? 0u : ((p.sig << sh) & 0x7fu);
  else
    part = -sh >= 32 ? 0u : ((p.sig >> (-sh)) & 0x7fu);
  return p.neg ? -static_cast<int>(part) : static_cast<int>(part);
}

// S[j][x][l] (int8) for x < np, l < kp and j below the slice count of x's
// 64-row block (at most S7MAX): slice j of the operand value (x, l) (A row x or
// B column x, reduction index l; the bias index as in path 2), zero past the
// operand. A workgroup converts a 64 x 64 block, read along the source's
// contiguous dimension (16-byte pieces where the operand allows) into LDS, and
// writes each slice's 16 bytes per thread.
typedef uint16_t Raw7_t[64][72];   // [x][l]; 144-byte rows

template <typename E, bool IS_A, bool RC>
__device__ inline void slice7_prep_block(const GemmArgs& g, const int* __restrict__ top, const int* __restrict__ low,
                                         int64_t n, int64_t np, int64_t kp, int8_t* __restrict__ S, int64_t blk,
                                         Raw7_t& raw, int& nsl) {
  using T = typename E::T;
  const int tid = threadIdx.x;
  const int64_t lb = kp / 64;
  const int64_t x0 = blk / lb * 64, l0 = blk % lb * 64;
  const int64_t kt = g.red + (g.bias ? 1 : 0);
  const T* X = static_cast<const T*>(IS_A ? g.A : g.B);
  const int64_t ld = IS_A ? g.lda : g.ldb;
  if (tid == 0) nsl = 0;
  __syncthreads();
  // the slices of this 64-row block (the tile's count on that side)
  if (tid < 64 && x0 + tid < n) atomicMax(&nsl, slices7_of(top[x0 + tid], low[x0 + tid]));
  if (X && (IS_A ? g.vec_a : g.vec_b) && x0 + 64 <= n && l0 + 64 <= g.red) {
    // 16-byte pieces along the contiguous dimension
    for (int i = tid; i < 512; i += 256) {
      if constexpr (RC) {
        const int x = i >> 3, pc = i & 7;
        *reinterpret_cast<uint4*>(&raw[x][8 * pc]) = *reinterpret_cast<const uint4*>(X + (x0 + x) * ld + l0 + 8 * pc);
      } else {
        const int l = i >> 3, pc = i & 7;
        const uint4 v = *reinterpret_cast<const uint4*>(X + (l0 + l) * ld + x0 + 8 * pc);
        const uint16_t* e = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
        for (int q = 0; q < 8; ++q) raw[8 * pc + q][l] = e[q];
      }
    }
  } else {
    for (int i = tid; i < 64 * 64; i += 256) {
      const int fast = i % 64, slow = i / 64;
      const int x = RC ? slow : fast, l = RC ? fast : slow;
      const int64_t gx = x0 + x, gl = l0 + l;
      uint16_t v = 0;
      if (gx < n && gl < g.red && X) {
        const T e = RC ? X[gx * ld + gl] : X[gl * ld + gx];
        __builtin_memcpy(&v, &e, 2);
      }
      raw[x][l] = v;
    }
  }
  __syncthreads();
  // thread: row x = tid / 4, the 16 reduction indices from 16 (tid % 4); each
  // slice's 16 bytes in one store, slices past the block's count not written
  // (the int8 kernel reads no further)
  const int nw = nsl < S7MAX ? nsl : S7MAX;
  const int x = tid >> 2, lq = (tid & 3) * 16;
  const int64_t gx = x0 + x;
  const int t = gx < n ? top[gx] : 0;
  uint32_t w[S7MAX][4];
#pragma unroll
  for (int j = 0; j < S7MAX; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c) w[j][c] = 0;
  uint16_t rv[16];
  *reinterpret_cast<uint4*>(&rv[0]) = *reinterpret_cast<const uint4*>(&raw[x][lq]);
  *reinterpret_cast<uint4*>(&rv[8]) = *reinterpret_cast<const uint4*>(&raw[x][lq + 8]);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t gl = l0 + lq + i;
    if (gx < n && gl < kt) {
      Parts p;
      if (gl == g.red || (IS_A && !X)) {
        p = IS_A ? a_at<E, RC>(g, gx, gl) : b_at<E, RC>(g, gl, gx);
      } else {
        T e;
        __builtin_memcpy(&e, &rv[i], 2);
        p = parts<E>(e);
      }
      if (p.finite && p.sig) {
        // the value in units of 2^(t - 7 S7MAX + 1): slice j is bits 7 (S7MAX - 1 - j) .. + 6
        // (the same as slice7(p, t, j); bits below the last slice drop out in both)
        const int sh = p.lsb - (t - S7 * S7MAX + 1);
        const uint64_t m = sh >= 0 ? static_cast<uint64_t>(p.sig) << sh
                                   : static_cast<uint64_t>(p.sig) >> (-sh < 63 ? -sh : 63);
        const uint32_t neg = p.neg ? 0xffu : 0u;
#pragma unroll
        for (int j = 0; j < S7MAX; ++j) {
          const uint32_t part = static_cast<uint32_t>(m >> (S7 * (S7MAX - 1 - j))) & 0x7fu;
          w[j][i >> 2] |= (((part ^ neg) + (neg & 1u)) & 0xffu) << (8 * (i & 3));
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < S7MAX; ++j)
    if (j < nw)
      *reinterpret_cast<uint4*>(S + (j * np + gx) * kp + l0 + lq) = uint4{w[j][0], w[j][1], w[j][2], w[j][3]};
}

// both operands in one launch: blocks below blocks_a convert A, the rest B
template <typename E, bool A_RC, bool B_RC>
__global__ void __launch_bounds__(256) slice7_prep_kernel(GemmArgs g, Stats st, int64_t npa, int64_t npb, int64_t kp,
                                                          int8_t* __restrict__ SA, int8_t* __restrict__ SB,
                                                          int64_t blocks_a) {
  __shared__ __attribute__((aligned(16))) Raw7_t raw;
  __shared__ int nsl;
  const int64_t b = blockIdx.x;
  if (b < blocks_a)
    slice7_prep_block<E, true, A_RC>(g, st.topA, st.lowA, g.rows, npa, kp, SA, b, raw, nsl);
  else
    slice7_prep_block<E, false, B_RC>(g, st.topB, st.lowB, g.cols, npb, kp, SB, b - blocks_a, raw, nsl);
}

typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef int v16i_t __attribute__((ext_vector_type(16)));
typedef uint32_t v4u_rs __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// buffer resource: base address, stride 0, size in bytes (reads past it return zeros)
__device__ inline v4u_rs rsrc_of(const void* src, int64_t bytes) {
  const uint64_t base = reinterpret_cast<uint64_t>(src);
  return v4u_rs{static_cast<uint32_t>(base), static_cast<uint32_t>(base >> 32) & 0xffffu, static_cast<uint32_t>(bytes),
                0x00020000u};
}

// LDS stage of one slice: 64 rows (or columns) x 128 reduction indices, row x
// in 128 bytes with 16-byte piece p in slot p XOR sw7(x), so that the fragment
// reads of 32 rows at one piece spread over the banks.
__device__ inline int sw7(int x) { return ((x >> 1) & 7) ^ ((x >> 3) & 1); }

typedef int8_t Ls7_t[2][2 * S7MAX][64 * K7];

// One tile whose rows need LA and columns LB slices (both at least 1), with
// the counts fixed at compile time so that the fragment reads and the LA x LB
// matrix instructions of a step are one straight block the compiler can
// schedule freely. Eight waves in a 4 x 2 grid, 16 x 32 outputs each as two
// 16 x 16 blocks: acc = MFMA(B fragment, A fragment, acc) with
// V_MFMA_I32_16X16X64_I8, the lane holding row lane % 16 and, in accumulator e
// of block b, column 16 b + 4 (lane / 16) + e. Fragments: lane l holds 16 bytes
// of its row (column) at reduction indices 64 k64 + 16 (l / 16) .. + 15, the
// same map for A and B, so the products pair up.
//
// base: the LDS buffer of the tile's first stage; have0: that stage is already
// staged (requested by the previous tile's loader waves). pf: during its last
// stage the tile requests the first stage of the next tile (rows from nr0,
// columns from nc0, nLA and nLB slices) into the other buffer. Returns that
// buffer, or -1 when nothing was requested.
template <typename O, int LA, int LB>
__device__ __forceinline__ int sliced7_tile(const GemmArgs& g, const Stats& st, Ls7_t& Ls, int64_t r0, int64_t c0,
                                            const int8_t* SA, const int8_t* SB, int64_t npa, int64_t npb, int64_t kp,
                                            int64_t sa_bytes, int64_t sb_bytes, int base, bool have0, bool pf,
                                            int64_t nr0, int64_t nc0, int nLA, int nLB) {
  constexpr int NQ = LA + LB - 1;   // weight classes q = s + t
  constexpr int QMAX = NQ - 1;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = (wave >> 1) * 16, wn = (wave & 1) * 32;
  const int fr = lane & 15, fq = lane >> 4;
  const int xa = wm + fr, xb0 = wn + fr, xb1 = wn + 16 + fr;
  // the output scales' top bits, fetched now so that their latency hides behind the loop
  const int64_t ro = r0 + wm + fr;
  const int ta = ro < g.rows ? st.topA[ro] : 0;
  int tb[2][4];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t c = c0 + wn + 16 * b + 4 * fq + e;
      tb[b][e] = c < g.cols ? st.topB[c] : 0;
    }

  __int128 Z[8];
  v4i_t acc[NQ][2];
#pragma unroll
  for (int i = 0; i < 8; ++i) Z[i] = 0;
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[q][b] = v4i_t{0, 0, 0, 0};
  const int nks = static_cast<int>(kp / K7);

  // Staging by direct-to-LDS buffer loads: a slice's 64 x 128 stage is eight 1 KB
  // wave instructions, instruction gi putting rows 8 gi .. 8 gi + 7 in place, lane
  // l fetching the piece that belongs at byte 16 l (row 8 gi + l / 8, slot l % 8).
  // The lane's byte offset depends on gi only; the slice and the stage go into
  // the scalar offset.
  const v4u_rs rsa = rsrc_of(SA, sa_bytes), rsb = rsrc_of(SB, sb_bytes);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t sla = static_cast<uint32_t>(npa * kp), slb = static_cast<uint32_t>(npb * kp);
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)&Ls[0][0][0]));
  auto voff = [&](int64_t base, int gi) {
    const int x = 8 * gi + (lane >> 3);
    return static_cast<uint32_t>((base + x) * kp + 16 * ((lane & 7) ^ sw7(x)));
  };
  // instruction gi of slice j (la A slices, then B slices) of stage ks into buffer b
  auto issue = [&](int j, int la, int gi, uint32_t va, uint32_t vb, int ks, int b) {
    const bool is_a = j < la;
    const int sl = is_a ? j : j - la;
    const uint32_t so = static_cast<uint32_t>(sl) * (is_a ? sla : slb) + static_cast<uint32_t>(ks) * K7;
    const uint32_t m0 =
        lds0 + static_cast<uint32_t>(b * 2 * S7MAX + (is_a ? sl : S7MAX + sl)) * (64 * K7) + 1024u * static_cast<uint32_t>(gi);
    if (is_a)
      __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                       :
                       : "s"(m0), "v"(va), "s"(rsa), "s"(so)
                       : "memory", "m0");
    else
      __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                       :
                       : "s"(m0), "v"(vb), "s"(rsb), "s"(so)
                       : "memory", "m0");
  };
  // The first stage: wave w issues instruction w of every slice. The later ones:
  // waves 0 .. 3 (one on each SIMD) issue instructions 2 w and 2 w + 1 of every
  // slice of stage ks + 1 at the start of stage ks, while the other wave on
  // their SIMD goes straight to the matrix work.
  const bool loader = wave_u < 4;
  const uint32_t va0 = voff(r0, 2 * wave_u), va1 = voff(r0, 2 * wave_u + 1);
  const uint32_t vb0 = voff(c0, 2 * wave_u), vb1 = voff(c0, 2 * wave_u + 1);

  if (!have0 && nks > 0) {
    const uint32_t va = voff(r0, wave_u), vb = voff(c0, wave_u);
#pragma unroll
    for (int j = 0; j < LA + LB; ++j) issue(j, LA, wave_u, va, vb, 0, base);
  }
  __builtin_amdgcn_s_waitcnt(0);   // this wave's loads are in LDS
  __asm__ volatile("" ::: "memory");
  __syncthreads();
  const bool pf_here = pf && nks > 0;
  auto stage = [&](int ks, auto with_loads) {
    constexpr bool WL = decltype(with_loads)::value;
    const int buf = (ks + base) & 1;
    // the next stage goes into the other buffer, read last in the previous stage
    if (WL && loader) {
#pragma unroll
      for (int j = 0; j < LA + LB; ++j) {
        issue(j, LA, 2 * wave_u, va0, vb0, ks + 1, buf ^ 1);
        issue(j, LA, 2 * wave_u + 1, va1, vb1, ks + 1, buf ^ 1);
      }
    }
    // the last stage requests the next tile's first stage
    if (!WL && pf_here && loader) {
      const uint32_t na0 = voff(nr0, 2 * wave_u), na1 = voff(nr0, 2 * wave_u + 1);
      const uint32_t nb0 = voff(nc0, 2 * wave_u), nb1 = voff(nc0, 2 * wave_u + 1);
      for (int j = 0; j < nLA + nLB; ++j) {
        issue(j, nLA, 2 * wave_u, na0, nb0, 0, buf ^ 1);
        issue(j, nLA, 2 * wave_u + 1, na1, nb1, 0, buf ^ 1);
      }
    }
    // Both 64-index steps' fragments are read up front, the second step's
    // between the first step's matrix instructions (two per read), so that the
    // LDS latency is paid once per stage.
    const int8_t* lsb = &Ls[buf][0][0];
    v4i_t af[2][LA], bf[2][LB][2];
#pragma unroll
    for (int k64 = 0; k64 < K7 / 64; ++k64) {
      const int pc = 4 * k64 + fq;
      const int oa = xa * K7 + 16 * (pc ^ sw7(xa));
      const int ob0 = xb0 * K7 + 16 * (pc ^ sw7(xb0)), ob1 = xb1 * K7 + 16 * (pc ^ sw7(xb1));
#pragma unroll
      for (int s = 0; s < LA; ++s) af[k64][s] = *reinterpret_cast<const v4i_t*>(lsb + s * (64 * K7) + oa);
#pragma unroll
      for (int t = 0; t < LB; ++t) {
        const int8_t* bt = lsb + (S7MAX + t) * (64 * K7);
        bf[k64][t][0] = *reinterpret_cast<const v4i_t*>(bt + ob0);
        bf[k64][t][1] = *reinterpret_cast<const v4i_t*>(bt + ob1);
      }
    }
#pragma unroll
    for (int k64 = 0; k64 < K7 / 64; ++k64)
#pragma unroll
      for (int t = 0; t < LB; ++t)
#pragma unroll
        for (int s = 0; s < LA; ++s) {
          acc[s + t][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bf[k64][t][0], af[k64][s], acc[s + t][0], 0, 0, 0);
          acc[s + t][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bf[k64][t][1], af[k64][s], acc[s + t][1], 0, 0, 0);
        }
    {
      constexpr int NR = LA + 2 * LB;    // fragment reads per step
      constexpr int NM = 2 * LA * LB;    // matrix instructions per step
      __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
      constexpr int NI = NR <= NM / 2 ? NR : NM / 2;   // second-step reads placed two instructions apart
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if constexpr (NR > NI) __builtin_amdgcn_sched_group_barrier(0x100, NR - NI, 0);
      constexpr int REM = 2 * NM - 2 * NI;
      __builtin_amdgcn_sched_group_barrier(0x008, REM, 0);
    }
    if (ks % FL7 == FL7 - 1 || ks == nks - 1) {
      // The exact int32 sums of every class, weighted 2^(7 (QMAX - q)): the five
      // lowest weights (up to 2^28) sum in an int64 below 2^60, the four highest
      // (2^35 up) in an int64 below 2^53 counted in units of 2^35; one int128 add.
      int64_t lo[8], hi[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) lo[i] = hi[i] = 0;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int sh = S7 * (QMAX - q);
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t v = acc[q][b][e];
            if (sh < 5 * S7)
              lo[4 * b + e] += v << sh;
            else
              hi[4 * b + e] += v << (sh - 5 * S7);
            acc[q][b][e] = 0;
          }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) Z[i] += (static_cast<__int128>(hi[i]) << (5 * S7)) + lo[i];
    }
    if constexpr (WL) {
      __builtin_amdgcn_s_waitcnt(0);   // this wave's requests for the next stage are in LDS
      __asm__ volatile("" ::: "memory");
    }
    // (every wave's requests are in) and every wave is done reading this stage;
    // the next tile's first stage stays in flight through the rounding below
    __syncthreads();
  };
  for (int ks = 0; ks + 1 < nks; ++ks) stage(ks, std::true_type{});
  if (nks > 0) stage(nks - 1, std::false_type{});

  using OT = typename O::T;
  OT* out = static_cast<OT*>(g.out);
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t c = c0 + wn + 16 * b + 4 * fq + e;
      if (ro < g.rows && c < g.cols) {
        const __int128 z = Z[4 * b + e];
        const double v = z == 0 ? 0.0 : round_odd53(z, ta + tb[b][e] - 2 * (S7 - 1) - S7 * QMAX);
        out[ro * g.cols + c] = round_from_f64<O>(v);
      }
    }
  return pf_here ? (((nks - 1 + base) & 1) ^ 1) : -1;
}

// A tile's slice counts (LA, LB) and whether it goes elsewhere (ew), from
// every wave alike (lane i looks at row r0 + i and column c0 + i).
__device__ inline void tile7_info(const GemmArgs& g, const Stats& st, int tile, int tiles_c, int enabled, int& LA,
                                  int& LB, int& ew) {
  const int lane = threadIdx.x & 63;
  const int64_t r0 = static_cast<int64_t>(tile / tiles_c) * TILE, c0 = static_cast<int64_t>(tile % tiles_c) * TILE;
  int la = 0, lb = 0, bad = 0;
  if (r0 + lane < g.rows) {
    la = slices7_of(st.topA[r0 + lane], st.lowA[r0 + lane]);
    bad |= st.badA[r0 + lane];
  }
  if (c0 + lane < g.cols) {
    lb = slices7_of(st.topB[c0 + lane], st.lowB[c0 + lane]);
    bad |= st.badB[c0 + lane];
  }
  for (int o = 32; o > 0; o >>= 1) {
    la = max(la, __shfl_xor(la, o));
    lb = max(lb, __shfl_xor(lb, o));
    bad |= __shfl_xor(bad, o);
  }
  LA = __builtin_amdgcn_readfirstlane(la);
  LB = __builtin_amdgcn_readfirstlane(lb);
  ew = (!enabled || __builtin_amdgcn_readfirstlane(bad) != 0 || LA > S7MAX || LB > S7MAX) ? 1 : 0;
}

// Persistent: workgroup b takes tiles b, b + G, b + 2 G, ... (G workgroups,
// one per compute unit), each tile's first stage staged during the previous
// tile's last stage where both take this path.
template <typename O>
__global__ void __launch_bounds__(512, 2) sliced7_kernel(GemmArgs g, Stats st, int tiles_c, int tiles,
                                                         const int8_t* __restrict__ SA, const int8_t* __restrict__ SB,
                                                         int64_t npa, int64_t npb, int64_t kp, int64_t sa_bytes,
                                                         int64_t sb_bytes, int enabled) {
  // two stages (double buffered) of A slices, then B slices
  __shared__ __attribute__((aligned(16))) Ls7_t Ls;
  const int tid = threadIdx.x;
  int base = 0;
  bool have0 = false;
  int LA, LB, ew;
  tile7_info(g, st, blockIdx.x, tiles_c, enabled, LA, LB, ew);
  for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    if (tid == 0) {
      st.flag[tile] = ew;
      if (ew) atomicAdd(&st.left[0], 1);
    }
    const int64_t r0 = static_cast<int64_t>(tile / tiles_c) * TILE, c0 = static_cast<int64_t>(tile % tiles_c) * TILE;
    const int nt = tile + gridDim.x;
    int nLA = 0, nLB = 0, nEW = 1;
    if (nt < tiles) tile7_info(g, st, nt, tiles_c, enabled, nLA, nLB, nEW);
    const bool pf = !nEW && nLA > 0 && nLB > 0;
    const int64_t nr0 = static_cast<int64_t>(nt / tiles_c) * TILE, nc0 = static_cast<int64_t>(nt % tiles_c) * TILE;
    int nb = -1;
    if (!ew && (LA == 0 || LB == 0)) {   // an all-zero row or column block: every product is zero
      using OT = typename O::T;
      OT* out = static_cast<OT*>(g.out);
      for (int i = tid; i < TILE * TILE; i += 512) {
        const int64_t r = r0 + i / TILE, c = c0 + i % TILE;
        if (r < g.rows && c < g.cols) out[r * g.cols + c] = round_from_f64<O>(0.0);
      }
    } else if (!ew) {
      static_assert(S7MAX == 5, "one case per slice-count pair below");
      switch (LA * 8 + LB) {
#define DET_CR7_CASE(a, b)                                                                                   \
  case (a) * 8 + (b):                                                                                        \
    nb = sliced7_tile<O, a, b>(g, st, Ls, r0, c0, SA, SB, npa, npb, kp, sa_bytes, sb_bytes, base, have0, pf, \
                               nr0, nc0, nLA, nLB);                                                          \
    break;
#define DET_CR7_ROW(a) DET_CR7_CASE(a, 1) DET_CR7_CASE(a, 2) DET_CR7_CASE(a, 3) DET_CR7_CASE(a, 4) DET_CR7_CASE(a, 5)
        DET_CR7_ROW(1) DET_CR7_ROW(2) DET_CR7_ROW(3) DET_CR7_ROW(4) DET_CR7_ROW(5)
#undef DET_CR7_ROW
#undef DET_CR7_CASE
        default:
          break;
      }
    }
    have0 = nb >= 0;
    base = nb >= 0 ? nb : 0;
    LA = nLA;
    LB = nLB;
    ew = nEW;
  }
}

// ---- 2c. 8-bit slices, one pair at a time (16-bit inputs) --------------------
//
// The tiles that 2b leaves, from 8-bit slices on the bf16 pipe. A value of
// row r is cut into 8-bit slices below top_r: slice j holds the bits with
// weights 2^(top_r - 8 j - 7) .. 2^(top_r - 8 j) as a signed integer of
// magnitude below 2^8, which bf16 holds exactly. For one slice pair (s, t) the
// products are integers below 2^16 and V_MFMA_F32_32X32X16_BF16 sums them in
// float32; over 256 reduction indices every partial sum stays below
// 256 * 255^2 < 2^24, so the sum is exact whatever order the instruction adds
// in. Each 256-index sum is added to a float64 per weight class q = s + t (an
// integer below 2^53 for any reduction this tier takes); at the end of a class
// the float64 goes into the int128 at 8 (qmax - q) bits up, and the int128 is
// rounded as in 2. A tile flagged by 2b is taken here when its rows and columns
// need at most S8MAX slices (spans of at most 40 bits) and all its values are
// finite; the others stay flagged for path 2.
constexpr int S8 = 8;           // bits per slice
constexpr int S8MAX = 5;        // slices per value on this path
constexpr int K8 = 64;          // reduction indices per stage
constexpr int CH8 = 4;          // stages per exact float32 sum (256 indices)

__device__ inline int slices8_of(int t, int lo) { return t == NOBITS ? 0 : (t - lo + S8) / S8; }

// Slice j of a value whose row or column has top bit `top`, as a signed integer.
__device__ inline int slice8(const Parts& p, int top, int j) {
  if (p.sig == 0) return 0;
  const int low = top - S8 * j - (S8 - 1);
  const int sh = p.lsb - low;
  uint32_t part;
  if (sh >= 0)
    part = sh >= S8 ? 0u : ((p.sig << sh) & 0xffu);
  else
    part = -sh >= 32 ? 0u : ((p.sig >> (-sh)) & 0xffu);
  return p.neg ? -static_cast<int>(part) : static_cast<int>(part);
}

// bf16 bits of a small integer (exact: at most 8 significant bits)
__device__ inline uint16_t bf16_of_int(int v) {
  return static_cast<uint16_t>(__float_as_uint(static_cast<float>(v)) >> 16);
}

// S[j][x][l] (bf16 bits) for j < S8MAX, x < np, l < kp: slice j of the operand
// value (x, l) (A row x or B column x, reduction index l; the bias index as in
// path 2), zero past the operand. A workgroup converts a 64 x 64 block, read
// along the source's contiguous dimension through LDS and written along l.
typedef uint16_t Raw8_t[64][65];

template <typename E, bool IS_A, bool RC>
__device__ inline void slice8_prep_block(const GemmArgs& g, const int* __restrict__ top, int64_t n, int64_t np,
                                         int64_t kp, uint16_t* __restrict__ S, int64_t blk, Raw8_t& raw) {
  using T = typename E::T;
  const int tid = threadIdx.x;
  const int64_t lb = kp / 64;
  const int64_t x0 = blk / lb * 64, l0 = blk % lb * 64;
  const int64_t kt = g.red + (g.bias ? 1 : 0);
  const T* X = static_cast<const T*>(IS_A ? g.A : g.B);
  const int64_t ld = IS_A ? g.lda : g.ldb;
  // element (x, l) of the operand sits at x * ld + l (RC) or l * ld + x; the bias
  // index and an absent A are not read from memory (a_at / b_at below)
  for (int i = tid; i < 64 * 64; i += 256) {
    const int fast = i % 64, slow = i / 64;
    const int x = RC ? slow : fast, l = RC ? fast : slow;
    const int64_t gx = x0 + x, gl = l0 + l;
    uint16_t v = 0;
    if (gx < n && gl < g.red && X) {
      const T e = RC ? X[gx * ld + gl] : X[gl * ld + gx];
      __builtin_memcpy(&v, &e, 2);
    }
    raw[x][l] = v;
  }
  __syncthreads();
  for (int i = tid; i < 64 * 64; i += 256) {
    const int x = i / 64, l = i % 64;
    const int64_t gx = x0 + x, gl = l0 + l;
    int v[S8MAX];
#pragma unroll
    for (int j = 0; j < S8MAX; ++j) v[j] = 0;
    if (gx < n && gl < kt) {
      Parts p;
      if (gl == g.red || (IS_A && !X)) {
        p = IS_A ? a_at<E, RC>(g, gx, gl) : b_at<E, RC>(g, gl, gx);
      } else {
        T e;
        const uint16_t bits = raw[x][l];
        __builtin_memcpy(&e, &bits, 2);
        p = parts<E>(e);
      }
      if (p.finite && p.sig) {
        const int t = top[gx];
#pragma unroll
        for (int j = 0; j < S8MAX; ++j) v[j] = slice8(p, t, j);
      }
    }
#pragma unroll
    for (int j = 0; j < S8MAX; ++j) S[(j * np + gx) * kp + gl] = bf16_of_int(v[j]);
  }
}

// both operands in one launch: blocks below blocks_a convert A, the rest B
template <typename E, bool A_RC, bool B_RC>
__global__ void __launch_bounds__(256) slice8_prep_kernel(GemmArgs g, Stats st, int64_t npa, int64_t npb, int64_t kp,
                                                          uint16_t* __restrict__ SA, uint16_t* __restrict__ SB,
                                                          int64_t blocks_a) {
  __shared__ Raw8_t raw;
  if (st.left[0] == 0) return;   // the int8 path left no tile (uniform over the grid)
  const int64_t b = blockIdx.x;
  if (b < blocks_a)
    slice8_prep_block<E, true, A_RC>(g, st.topA, g.rows, npa, kp, SA, b, raw);
  else
    slice8_prep_block<E, false, B_RC>(g, st.topB, g.cols, npb, kp, SB, b - blocks_a, raw);
}

typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));

// LDS stage of one operand: 64 rows (or columns) x 64 reduction indices, row x
// in 128 bytes with 16-byte piece p in slot p XOR sw(x), so that the fragment
// reads of 32 rows at one piece spread over the banks.
__device__ inline int sw8(int x) { return ((x >> 1) & 7) ^ ((x >> 3) & 1); }

template <typename O>
__global__ void __launch_bounds__(256) sliced8_kernel(GemmArgs g, Stats st, int tiles_c,
                                                      const uint16_t* __restrict__ SA, const uint16_t* __restrict__ SB,
                                                      int64_t npa, int64_t npb, int64_t kp) {
  __shared__ __attribute__((aligned(16))) uint16_t Ls[2][2][64 * 64];   // [buffer][A, B][row * 64 + index]
  __shared__ int red_s[4];
  const int tid = threadIdx.x;
  const int tile = blockIdx.x;
  if (!st.flag[tile]) return;   // finished by 2b (uniform over the workgroup)
  const int64_t r0 = static_cast<int64_t>(tile / tiles_c) * TILE, c0 = static_cast<int64_t>(tile % tiles_c) * TILE;
  if (tid < 4) red_s[tid] = 0;
  __syncthreads();
  {
    const int i = tid & 63;
    if (tid < 64 && r0 + i < g.rows) {
      atomicMax(&red_s[0], slices8_of(st.topA[r0 + i], st.lowA[r0 + i]));
      if (st.badA[r0 + i]) atomicOr(&red_s[2], 1);
    } else if (tid >= 64 && tid < 128 && c0 + i < g.cols) {
      atomicMax(&red_s[1], slices8_of(st.topB[c0 + i], st.lowB[c0 + i]));
      if (st.badB[c0 + i]) atomicOr(&red_s[2], 1);
    }
  }
  __syncthreads();
  const int LA = red_s[0], LB = red_s[1];
  const bool elsewhere = red_s[2] || LA > S8MAX || LB > S8MAX;
  if (tid == 0) {
    st.flag[tile] = elsewhere ? 1 : 0;
    if (elsewhere) atomicAdd(&st.left[1], 1);
  }
  if (elsewhere) return;   // uniform over the workgroup

  // a wave owns 32 x 32 outputs; acc = MFMA(B fragment, A fragment, acc): the
  // lane holds row lane % 32 and, in accumulator 4 q + e, column 8 q + 4 (lane / 32) + e
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  const int fr = lane & 31, fh = lane >> 5;

  __int128 Z[16];
  double C[16];
  v16f_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) { Z[i] = 0; C[i] = 0.0; acc[i] = 0.0f; }

  const int nks = static_cast<int>(kp / K8);
  const int qmax = LA + LB - 2;
  const int64_t nsteps = LA > 0 && LB > 0 ? static_cast<int64_t>(LA) * LB * nks : 0;
  // step state: class q, slice s of A (t = q - s of B), stage ks
  auto smin = [&](int q) { return q - (LB - 1) > 0 ? q - (LB - 1) : 0; };
  auto smax = [&](int q) { return q < LA - 1 ? q : LA - 1; };
  // the thread's two 16-byte pieces of each operand per stage: rows x0, x1 = x0 + 32, piece pc
  const int x0 = tid >> 3, x1 = x0 + 32, pc0 = tid & 7;
  const int la0 = x0 * 64 + 8 * (pc0 ^ sw8(x0)), la1 = x1 * 64 + 8 * (pc0 ^ sw8(x1));
  const uint16_t* ga = SA + (r0 + x0) * kp + 8 * pc0;   // slice 0, stage 0
  const uint16_t* gb = SB + (c0 + x0) * kp + 8 * pc0;
  const int64_t sa_step = npa * kp, sb_step = npb * kp, half = 32 * kp;
  uint4 ra0 = {}, ra1 = {}, rb0 = {}, rb1 = {};
  // fragment reads: row (column) wm + fr (wn + fr), piece 2 k16 + fh of the stage
  const int xa = wm + fr, xb = wn + fr;

  int q = 0, s = 0, ks = 0;
  if (nsteps > 0) {
    const uint16_t* pa = ga;
    const uint16_t* pb = gb + static_cast<int64_t>(q - s) * sb_step;
    ra0 = *reinterpret_cast<const uint4*>(pa);
    ra1 = *reinterpret_cast<const uint4*>(pa + half);
    rb0 = *reinterpret_cast<const uint4*>(pb);
    rb1 = *reinterpret_cast<const uint4*>(pb + half);
    *reinterpret_cast<uint4*>(&Ls[0][0][la0]) = ra0;
    *reinterpret_cast<uint4*>(&Ls[0][0][la1]) = ra1;
    *reinterpret_cast<uint4*>(&Ls[0][1][la0]) = rb0;
    *reinterpret_cast<uint4*>(&Ls[0][1][la1]) = rb1;
  }
  __syncthreads();
  for (int64_t n = 0; n < nsteps; ++n) {
    const int buf = static_cast<int>(n & 1);
    // the next step's (class, slice, stage)
    int nq = q, ns = s, nk = ks + 1;
    if (nk == nks) {
      nk = 0;
      ++ns;
      if (ns > smax(nq)) {
        ++nq;
        ns = smin(nq);
      }
    }
    const bool more = n + 1 < nsteps;
    if (more) {
      const uint16_t* pa = ga + ns * sa_step + static_cast<int64_t>(nk) * K8;
      const uint16_t* pb = gb + (nq - ns) * sb_step + static_cast<int64_t>(nk) * K8;
      ra0 = *reinterpret_cast<const uint4*>(pa);
      ra1 = *reinterpret_cast<const uint4*>(pa + half);
      rb0 = *reinterpret_cast<const uint4*>(pb);
      rb1 = *reinterpret_cast<const uint4*>(pb + half);
    }
    const uint16_t* la = &Ls[buf][0][0];
    const uint16_t* lb = &Ls[buf][1][0];
#pragma unroll
    for (int k16 = 0; k16 < K8 / 16; ++k16) {
      const int pc = 2 * k16 + fh;
      const v4u_t af = *reinterpret_cast<const v4u_t*>(la + xa * 64 + 8 * (pc ^ sw8(xa)));
      const v4u_t bf = *reinterpret_cast<const v4u_t*>(lb + xb * 64 + 8 * (pc ^ sw8(xb)));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf_t, bf), __builtin_bit_cast(v8bf_t, af), acc,
                                                    0, 0, 0);
    }
    const bool pair_end = ks == nks - 1;
    if (pair_end || ks % CH8 == CH8 - 1) {   // an exact 256-index sum (or the pair's last, shorter one)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        C[i] = C[i] + static_cast<double>(acc[i]);
        acc[i] = 0.0f;
      }
      if (pair_end && s == smax(q)) {   // the class is complete
        const int sh = S8 * (qmax - q);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          Z[i] += static_cast<__int128>(static_cast<int64_t>(C[i])) << sh;
          C[i] = 0.0;
        }
      }
    }
    if (more) {
      *reinterpret_cast<uint4*>(&Ls[buf ^ 1][0][la0]) = ra0;
      *reinterpret_cast<uint4*>(&Ls[buf ^ 1][0][la1]) = ra1;
      *reinterpret_cast<uint4*>(&Ls[buf ^ 1][1][la0]) = rb0;
      *reinterpret_cast<uint4*>(&Ls[buf ^ 1][1][la1]) = rb1;
    }
    __syncthreads();
    q = nq;
    s = ns;
    ks = nk;
  }

  using OT = typename O::T;
  OT* out = static_cast<OT*>(g.out);
  const int64_t r = r0 + wm + fr;
#pragma unroll
  for (int qq = 0; qq < 4; ++qq)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t c = c0 + wn + 8 * qq + 4 * fh + e;
      if (r < g.rows && c < g.cols) {
        const __int128 z = Z[4 * qq + e];
        const double v = z == 0 ? 0.0 : round_odd53(z, st.topA[r] + st.topB[c] - 2 * (S8 - 1) - S8 * qmax);
        out[r * g.cols + c] = round_from_f64<O>(v);
      }
    }
}

// ---- 3. fallback ---------------------------------------------------------------

// Adds the finite float64 term v to the chunks (each chunk counts 32 bits;
// the int64 leaves room for 2^31 additions before a carry is needed).
__device__ inline void sacc_add(int64_t* ch, double v) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const int e = static_cast<int>((u >> 52) & 0x7ffu);
  if (e == 0) return;   // zero (subnormal float64 terms do not occur: |products| >= 2^-298)
  const uint64_t M = (u & 0xfffffffffffffull) | (1ull << 52);   // |v| = M * 2^(e - 1075)
  const int bit = e - 1075 + OFF;
  const int ci = bit >> 5, sh = bit & 31;
  const unsigned __int128 w = static_cast<unsigned __int128>(M) << sh;
  const int64_t p0 = static_cast<int64_t>(static_cast<uint64_t>(w) & 0xffffffffu);
  const int64_t p1 = static_cast<int64_t>(static_cast<uint64_t>(w >> 32) & 0xffffffffu);
  const int64_t p2 = static_cast<int64_t>(static_cast<uint64_t>(w >> 64));
  if (u >> 63) {
    ch[ci] -= p0;
    ch[ci + 1] -= p1;
    ch[ci + 2] -= p2;
  } else {
    ch[ci] += p0;
    ch[ci + 1] += p1;
    ch[ci + 2] += p2;
  }
}

// The chunks' exact value rounded to odd at 53 bits (see round_odd53).
__device__ inline double sacc_round_odd53(int64_t* ch) {
  // carry-propagate into 32-bit digits; the final carry is the sign extension
  int64_t carry = 0;
  for (int i = 0; i < NCH; ++i) {
    const int64_t v = ch[i] + carry;
    ch[i] = v & 0xffffffff;
    carry = v >> 32;   // arithmetic shift
  }
  const bool neg = carry < 0;
  if (neg) {   // magnitude = two's complement of the digits
    int64_t c = 1;
    for (int i = 0; i < NCH; ++i) {
      const int64_t v = ((~ch[i]) & 0xffffffff) + c;
      ch[i] = v & 0xffffffff;
      c = v >> 32;
    }
  }
  int hi = -1;
  for (int i = NCH - 1; i >= 0; --i)
    if (ch[i]) {
      hi = i;
      break;
    }
  if (hi < 0) return 0.0;
  // the top 96 bits from three digits, and whether anything below them is set
  const uint64_t d2 = static_cast<uint64_t>(ch[hi]);
  const uint64_t d1 = hi >= 1 ? static_cast<uint64_t>(ch[hi - 1]) : 0;
  const uint64_t d0 = hi >= 2 ? static_cast<uint64_t>(ch[hi - 2]) : 0;
  bool sticky = false;
  for (int i = 0; i < hi - 2; ++i) sticky |= ch[i] != 0;
  const unsigned __int128 w = (static_cast<unsigned __int128>(d2) << 64) | (d1 << 32) | d0;   // < 2^96
  const int n = 64 - __builtin_clzll(d2) + 64;   // bit length of w
  const int sh = n - 53;                        // >= 12
  uint64_t top = static_cast<uint64_t>(w >> sh);
  if (sticky || (w & ((static_cast<unsigned __int128>(1) << sh) - 1)) != 0) top |= 1u;
  const int scale = 32 * (hi - 2) + sh - OFF;   // weight of top's last bit
  const double d = static_cast<double>(top) * pow2(scale);
  return neg ? -d : d;
}

template <typename E, typename O, bool A_RC, bool B_RC>
__global__ void __launch_bounds__(256) fallback_kernel(GemmArgs g, Stats st, int tiles_c) {
  __shared__ int64_t acc[256][NCH + 1];
  const int tile = blockIdx.x;
  if (!st.flag[tile]) return;   // uniform over the workgroup
  const int tid = threadIdx.x;
  const int64_t r0 = static_cast<int64_t>(tile / tiles_c) * TILE, c0 = static_cast<int64_t>(tile % tiles_c) * TILE;
  const int64_t kt = g.red + (g.bias ? 1 : 0);
  int64_t* ch = acc[tid];
  using OT = typename O::T;
  OT* out = static_cast<OT*>(g.out);
  const int64_t c = c0 + tid % 64;
  for (int q = 0; q < 16; ++q) {
    const int64_t r = r0 + tid / 64 + 4 * q;
    if (r >= g.rows || c >= g.cols) continue;
    for (int i = 0; i < NCH; ++i) ch[i] = 0;
    double nonfinite = 0.0;
    bool has_nf = false;
    for (int64_t l = 0; l < kt; ++l) {
      // the stored values, upcast exactly (A is a column of ones when absent)
      const typename E::T* A = static_cast<const typename E::T*>(g.A);
      const typename E::T* B = static_cast<const typename E::T*>(g.B);
      const double a = (l == g.red || !A) ? 1.0 : E::up(A_RC ? A[r * g.lda + l] : A[l * g.lda + r]);
      const double b = E::up(l == g.red ? static_cast<const typename E::T*>(g.bias)[c]
                                        : (B_RC ? B[c * g.ldb + l] : B[l * g.ldb + c]));
      const double p = a * b;   // exact: products of f32/bf16/f16 values fit float64
      if (!__builtin_isfinite(p)) {
        nonfinite = has_nf ? nonfinite + p : p;
        has_nf = true;
      } else {
        sacc_add(ch, p);
      }
    }
    const double v = has_nf ? nonfinite : sacc_round_odd53(ch);
    out[r * g.cols + c] = round_from_f64<O>(v);
  }
}

// ---- launch -----------------------------------------------------------------

template <typename E, typename O, bool A_RC, bool B_RC>
hipError_t launch_typed(const GemmArgs& a, int force_fallback, hipStream_t stream) {
  using T = typename E::T;
  const int64_t tiles_r = (a.rows + TILE - 1) / TILE, tiles_c = (a.cols + TILE - 1) / TILE;
  const int64_t tiles = tiles_r * tiles_c;
  if (tiles > INT_MAX || tiles_c > INT_MAX) return hipErrorInvalidConfiguration;
  const int64_t kt = a.red + (a.bias ? 1 : 0);
  const int64_t ktp = (kt + KB - 1) / KB * KB;
  const int64_t npa = tiles_r * TILE, npb = tiles_c * TILE;
  // the 8-bit path for 16-bit inputs (force_fallback: 1 the superaccumulator for
  // every tile, 2 path 2 for every tile)
  const bool use8 = sizeof(T) == 2 && force_fallback == 0;
  const int64_t kp8 = (kt + K8 - 1) / K8 * K8;
  const int64_t kp7 = (kt + K7 - 1) / K7 * K7;
  // workspace: int stats and flags, then (256-byte aligned) the float slices of A
  // and B, then the bf16 slices of A and B
  const size_t ints = static_cast<size_t>(3 * a.rows + 3 * a.cols + tiles + 2);
  const size_t off_slices = (ints * sizeof(int) + 255) / 256 * 256;
  const size_t sa_floats = static_cast<size_t>(2 * ktp * npa), sb_floats = static_cast<size_t>(2 * ktp * npb);
  const size_t off8 = off_slices + ((sa_floats + sb_floats) * sizeof(float) + 255) / 256 * 256;
  const size_t s8a = use8 ? static_cast<size_t>(S8MAX * npa * kp8) : 0, s8b = use8 ? static_cast<size_t>(S8MAX * npb * kp8) : 0;
  const size_t off7 = off8 + ((s8a + s8b) * sizeof(uint16_t) + 255) / 256 * 256;
  const size_t s7a = use8 ? static_cast<size_t>(S7MAX * npa * kp7) : 0, s7b = use8 ? static_cast<size_t>(S7MAX * npb * kp7) : 0;
  void* ws = nullptr;
  hipError_t e = stream_workspace(stream, off7 + s7a + s7b, &ws);
  if (e != hipSuccess) return e;
  int* p = static_cast<int*>(ws);
  float* SA = reinterpret_cast<float*>(static_cast<char*>(ws) + off_slices);
  float* SB = SA + sa_floats;
  uint16_t* SA8 = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + off8);
  uint16_t* SB8 = SA8 + s8a;
  int8_t* SA7 = reinterpret_cast<int8_t*>(static_cast<char*>(ws) + off7);
  int8_t* SB7 = SA7 + s7a;
  Stats st;
  int* topA = p;
  int* lowA = topA + a.rows;
  int* badA = lowA + a.rows;
  int* topB = badA + a.rows;
  int* lowB = topB + a.cols;
  int* badB = lowB + a.cols;
  int* flag = badB + a.cols;
  int* left = flag + tiles;
  st.topA = topA; st.lowA = lowA; st.badA = badA;
  st.topB = topB; st.lowB = lowB; st.badB = badB;
  st.flag = flag;
  st.left = left;
  const int64_t nmax = a.rows > a.cols ? a.rows : a.cols;
  hipLaunchKernelGGL((stats_init_kernel<E>), dim3(static_cast<unsigned>((nmax + 255) / 256)), dim3(256), 0, stream,
                     a.rows, a.cols, topA, lowA, badA, topB, lowB, badB, static_cast<const T*>(a.bias),
                     a.A ? 0 : 1, left);
  const int64_t strip = 256, strip_cols = 32;   // more strips for per-column stats (one thread each)
  auto stats = [&](const void* X, bool rc, int64_t n_idx, int64_t red, int64_t ld, int* top, int* low, int* bad) {
    // the array is [n_idx][ld] (rc) or [red][ld] (!rc); ld is its contiguous length
    constexpr int64_t V = 16 / sizeof(T);
    const bool vec = reinterpret_cast<uintptr_t>(X) % 16 == 0 && ld % V == 0 && (rc ? red : n_idx) % V == 0;
    if (vec && rc) {
      hipLaunchKernelGGL((stats_rows_vec_kernel<E>), dim3(static_cast<unsigned>((n_idx * 64 + 255) / 256)), dim3(256), 0,
                         stream, static_cast<const T*>(X), n_idx, red, ld, top, low, bad);
    } else if (vec) {
      const int64_t groups = (n_idx / V + 63) / 64;
      // strips of 16 rows, longer while the grid would exceed 2048 workgroups
      int64_t vstrip = 16;
      while (groups * ((red + vstrip - 1) / vstrip) > 2048) vstrip *= 2;
      hipLaunchKernelGGL((stats_cols_vec_kernel<E>),
                         dim3(static_cast<unsigned>(groups * ((red + vstrip - 1) / vstrip))), dim3(256), 0, stream,
                         static_cast<const T*>(X), red, n_idx, ld, vstrip, top, low, bad);
    } else if (rc) {
      const int64_t waves = n_idx * ((red + strip - 1) / strip);
      hipLaunchKernelGGL((stats_kernel<E, true>), dim3(static_cast<unsigned>((waves * 64 + 255) / 256)), dim3(256), 0,
                         stream, static_cast<const T*>(X), n_idx, ld, strip, top, low, bad);
    } else {
      const int64_t threads = ld * ((red + strip_cols - 1) / strip_cols);
      hipLaunchKernelGGL((stats_kernel<E, false>), dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0,
                         stream, static_cast<const T*>(X), red, ld, strip_cols, top, low, bad);
    }
  };
  if (a.A) stats(a.A, A_RC, a.rows, a.red, a.lda, topA, lowA, badA);
  stats(a.B, B_RC, a.cols, a.red, a.ldb, topB, lowB, badB);
  if (use8) {
    // 2b: the direct loads address the slices with 32-bit byte offsets
    const int on7 = s7a < (size_t(1) << 31) && s7b < (size_t(1) << 31) ? 1 : 0;
    hipLaunchKernelGGL((slice7_prep_kernel<E, A_RC, B_RC>), dim3(static_cast<unsigned>((npa + npb) / 64 * (kp7 / 64))),
                       dim3(256), 0, stream, a, st, npa, npb, kp7, SA7, SB7, npa / 64 * (kp7 / 64));
    // one workgroup per compute unit when that gives each at least four tiles
    const int64_t g7 = a.num_cu > 0 && 4 * a.num_cu <= tiles ? a.num_cu : tiles;
    hipLaunchKernelGGL((sliced7_kernel<O>), dim3(static_cast<unsigned>(g7)), dim3(512), 0, stream, a, st,
                       static_cast<int>(tiles_c), static_cast<int>(tiles), SA7, SB7, npa, npb, kp7,
                       static_cast<int64_t>(s7a), static_cast<int64_t>(s7b), on7);
    hipLaunchKernelGGL((slice8_prep_kernel<E, A_RC, B_RC>), dim3(static_cast<unsigned>((npa + npb) / 64 * (kp8 / 64))),
                       dim3(256), 0, stream, a, st, npa, npb, kp8, SA8, SB8, npa / 64 * (kp8 / 64));
    hipLaunchKernelGGL((sliced8_kernel<O>), dim3(static_cast<unsigned>(tiles)), dim3(256), 0, stream, a, st,
                       static_cast<int>(tiles_c), SA8, SB8, npa, npb, kp8);
  }
  {
    const int64_t blocks = (ktp * (npa + npb) + 255) / 256;
    hipLaunchKernelGGL((slice_prep_kernel<E, A_RC, B_RC>), dim3(static_cast<unsigned>(blocks < 8192 ? blocks : 8192)),
                       dim3(256), 0, stream, a, topA, topB, npa, npb, ktp, SA, SB, use8 ? left + 1 : nullptr);
  }
  hipLaunchKernelGGL((sliced_kernel<O>), dim3(static_cast<unsigned>(tiles)), dim3(256), 0, stream, a, st,
                     static_cast<int>(tiles_c), force_fallback == 1 ? 1 : 0, SA, SB, npa, npb, ktp, use8 ? 1 : 0);
  hipLaunchKernelGGL((fallback_kernel<E, O, A_RC, B_RC>), dim3(static_cast<unsigned>(tiles)), dim3(256), 0, stream, a,
                     st, static_cast<int>(tiles_c));
  return hipGetLastError();
}

template <typename E, typename O>
hipError_t launch_eo(Op op, const GemmArgs& a, int force_fallback, hipStream_t stream) {
  switch (op) {
    case OP_FWD: return launch_typed<E, O, true, false>(a, force_fallback, stream);
    case OP_DX: return launch_typed<E, O, true, true>(a, force_fallback, stream);
    case OP_DW: return launch_typed<E, O, false, false>(a, force_fallback, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace cr

hipError_t launch_cr(Op op, Dt dt, const GemmArgs& a, int force_fallback, hipStream_t stream) {
  switch (dt) {
    case DT_F32: return cr::launch_eo<F32, F32>(op, a, force_fallback, stream);
    case DT_BF16:
      return a.out_f32 ? cr::launch_eo<BF16, F32>(op, a, force_fallback, stream)
                       : cr::launch_eo<BF16, BF16>(op, a, force_fallback, stream);
    case DT_F16:
      return a.out_f32 ? cr::launch_eo<F16, F32>(op, a, force_fallback, stream)
                       : cr::launch_eo<F16, F16>(op, a, force_fallback, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace detgemm
