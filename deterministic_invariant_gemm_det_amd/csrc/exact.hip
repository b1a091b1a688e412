// Exact tier: float64 tiles of 32 with Neumaier compensation across tiles.
//
// Method (Carbon README, alia-carbon 0.2.0, "How It Works"): the reduction is
// split into tiles, operands are upcast to float64, and the tile results are
// combined with Kahan-Babushka-Neumaier compensation in a fixed order. For one
// output:
//     p_t = fma chain over the tile's indices in ascending order, from +0
//     (s, c) <- Neumaier(s, c, p_t) for t ascending, from (+0, +0)
//     r = s + c (+ bias), then one round-to-nearest-even to the output type.
//
// gfx950 mapping
//   * The fma chains run on the float64 matrix cores: V_MFMA_F64_16X16X4_F64
//     computes, for each of its 16x16 outputs, acc = fma(a_k, b_k, acc) for
//     its four k in ascending order, each step rounded to nearest even (checked
//     bit for bit against a sequential fma chain, subnormals, signed zeros and
//     ties included). Eight of them in k order, started from +0, are exactly one
//     tile's chain p_t.
//   * The Neumaier combine runs on the float64 vector ALU, once per tile and
//     output, and overlaps with the next tile's matrix-core work.
//   * Zero padding past the end of the reduction adds fma(0, 0, p) = p + 0,
//     which leaves p unchanged because a chain started from +0 is never -0.
//     So a short last tile is computed as a padded full tile with the same bits.
//   * Every output is computed the same way wherever it sits, so a row's bits do
//     not depend on the number of rows, the tile grid or the launch.
//
// Workgroup: 256 threads = 4 waves in 2x2, 64x64 outputs; each wave owns 32x32
// outputs as 2x2 blocks of 16x16. Operand tiles are staged in LDS as float64,
// laid out [reduction index][row or column], double buffered.

#include "common.hpp"

namespace detgemm {
namespace {

constexpr int KT = 32;        // the method's tile width along the reduction
constexpr int BM = 64;        // workgroup output rows
constexpr int BN = 64;        // workgroup output columns
constexpr int THREADS = 256;

typedef double v4d __attribute__((ext_vector_type(4)));

// Neumaier's update of the compensated pair (s, c) with one tile partial p.
// Both branches form the exact rounding error of s + p; the operand selection
// reproduces the branch on |s| >= |p| exactly, NaN comparisons included.
__device__ inline void neumaier_add(double& s, double& c, double p) {
  const double tt = s + p;
  const bool s_big = __builtin_fabs(s) >= __builtin_fabs(p);
  const double big = s_big ? s : p;
  const double small = s_big ? p : s;
  c = c + ((big - tt) + small);
  s = tt;
}

// Stage a 32-deep slice of an operand into LDS as float64, layout dst[l][x]
// for l < KT (reduction) and x < 64 (row of A or column of B).
//   red_contig: element (x, l) is src[(x0 + x) * ld + l0 + l]   (reduction contiguous)
//   otherwise : element (x, l) is src[(l0 + l) * ld + x0 + x]   (reduction-major)
// Out-of-range elements are stored as +0.
template <typename E, bool RED_CONTIG>
__device__ inline void stage(double* __restrict__ dst, const typename E::T* __restrict__ src, int64_t ld,
                             int64_t x0, int64_t xlen, int64_t l0, int64_t llen) {
  const int t = threadIdx.x;
  if (RED_CONTIG) {
    const int x = t >> 2;             // 64 rows x 4 threads
    const int lb = (t & 3) * 8;       // 8 consecutive reduction indices each
    const int64_t gx = x0 + x;
    const typename E::T* row = src + gx * ld + l0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int l = lb + j;
      double v = 0.0;
      if (gx < xlen && l0 + l < llen) v = E::up(row[l]);
      dst[l * BM + x] = v;
    }
  } else {
    const int l = t >> 3;             // 32 reduction rows x 8 threads
    const int xb = (t & 7) * 8;       // 8 consecutive columns each
    const int64_t gl = l0 + l;
    const typename E::T* row = src + gl * ld + x0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int x = xb + j;
      double v = 0.0;
      if (gl < llen && x0 + x < xlen) v = E::up(row[x]);
      dst[l * BN + x] = v;
    }
  }
}

template <typename E, bool A_RED_CONTIG, bool B_RED_CONTIG>
__global__ void __launch_bounds__(THREADS) exact_kernel(GemmArgs args) {
  __shared__ double As[2][KT * BM];
  __shared__ double Bs[2][KT * BN];

  const typename E::T* __restrict__ A = static_cast<const typename E::T*>(args.A);
  const typename E::T* __restrict__ B = static_cast<const typename E::T*>(args.B);
  const int64_t tiles_n = (args.cols + BN - 1) / BN;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) / tiles_n) * BM;
  const int64_t col0 = (static_cast<int64_t>(blockIdx.x) % tiles_n) * BN;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wm = (wave >> 1) * 32;
  const int wn = (wave & 1) * 32;
  const int lr = lane & 15;   // row (A) / column (B, D) inside a 16x16 block
  const int lk = lane >> 4;   // k inside a group of four

  double s[2][2][4], c[2][2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) { s[i][j][e] = 0.0; c[i][j][e] = 0.0; }

  const int64_t ntiles = (args.red + KT - 1) / KT;
  stage<E, A_RED_CONTIG>(As[0], A, args.lda, row0, args.rows, 0, args.red);
  stage<E, B_RED_CONTIG>(Bs[0], B, args.ldb, col0, args.cols, 0, args.red);
  __syncthreads();

  for (int64_t t = 0; t < ntiles; ++t) {
    const int buf = static_cast<int>(t & 1);
    if (t + 1 < ntiles) {
      stage<E, A_RED_CONTIG>(As[buf ^ 1], A, args.lda, row0, args.rows, (t + 1) * KT, args.red);
      stage<E, B_RED_CONTIG>(Bs[buf ^ 1], B, args.ldb, col0, args.cols, (t + 1) * KT, args.red);
    }
    const double* __restrict__ as = As[buf];
    const double* __restrict__ bs = Bs[buf];
    v4d p[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) p[i][j] = v4d{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int g = 0; g < KT / 4; ++g) {
      const int kr = (4 * g + lk);
      const double a0 = as[kr * BM + wm + lr];
      const double a1 = as[kr * BM + wm + 16 + lr];
      const double b0 = bs[kr * BN + wn + lr];
      const double b1 = bs[kr * BN + wn + 16 + lr];
      p[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, p[0][0], 0, 0, 0);
      p[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, p[0][1], 0, 0, 0);
      p[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, p[1][0], 0, 0, 0);
      p[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, p[1][1], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) neumaier_add(s[i][j][e], c[i][j][e], p[i][j][e]);
    __syncthreads();
  }

  typename E::T* __restrict__ Y = static_cast<typename E::T*>(args.out);
  const typename E::T* __restrict__ bias = static_cast<const typename E::T*>(args.bias);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = col0 + wn + 16 * j + lr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = row0 + wm + 16 * i + 4 * e + lk;
        if (row < args.rows && col < args.cols) {
          double r = s[i][j][e] + c[i][j][e];
          if (bias) r = r + E::up(bias[col]);
          Y[row * args.cols + col] = round_from_f64<E>(r);
        }
      }
    }
}

template <typename E, bool AC, bool BC>
hipError_t launch_typed(const GemmArgs& a, hipStream_t stream) {
  const int64_t blocks = ((a.cols + BN - 1) / BN) * ((a.rows + BM - 1) / BM);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((exact_kernel<E, AC, BC>), dim3(static_cast<unsigned>(blocks)), dim3(THREADS), 0, stream, a);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_op(Op op, const GemmArgs& a, hipStream_t stream) {
  switch (op) {
    case OP_FWD: return launch_typed<E, true, false>(a, stream);   // X[i][k], W[k][j]
    case OP_DX:  return launch_typed<E, true, true>(a, stream);    // dY[i][n], W[q][n]
    case OP_DW:  return launch_typed<E, false, false>(a, stream);  // X[i][q], dY[i][j]
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_exact(Op op, Dt dt, const GemmArgs& a, hipStream_t stream) {
  switch (dt) {
    case DT_F32: return launch_op<F32>(op, a, stream);
    case DT_BF16: return launch_op<BF16>(op, a, stream);
    case DT_F16: return launch_op<F16>(op, a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace detgemm
