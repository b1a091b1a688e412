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
// Facts the kernels rely on
//   * Zero padding past the end of the reduction adds fma(0, 0, p) = p + 0,
//     which leaves p unchanged because a chain started from +0 is never -0.
//     So a short last tile is computed as a padded full tile with the same bits.
//   * Neumaier's update adds to c the exact rounding error of s + p_t. Knuth's
//     branch-free TwoSum yields the same exact error for all finite operands,
//     and with f32/bf16/f16 inputs s and p_t are always finite (every partial is
//     far below the float64 range); a non-finite input makes both forms NaN.
//     So the kernels use TwoSum (7 float64 adds per output and tile).
//   * Every output is computed the same way wherever it sits, so a row's bits do
//     not depend on the number of rows, the tile grid or the launch.
//
// Three kernels implement it, with identical bits (the default is mfma4, in
// 64- or 48-row blocks by launch balance, and mfma16 for grids of at most two
// 64 x 64 blocks per compute unit):
//   mfma4 — the fma chains on V_MFMA_F64_4X4X4_4B_F64: four independent 4x4
//           blocks per instruction, each output acc = fma(a_k, b_k, acc) over
//           its four k in ascending order, one rounding per step (checked bit
//           for bit against a sequential fma chain, subnormals, signed zeros and
//           ties included). Eight of them in k order from +0 are one tile's chain.
//           On gfx950 this shape runs the float64 pipe at close to its peak
//           (about 1.5x the rate of the 16x16x4 shape). A wave owns 64 rows x 16
//           columns: four row fragments times the same 16 columns presented in
//           four block rotations, so that every (row, column) pair meets once.
//   mfma16 — the same on V_MFMA_F64_16X16X4_F64 (one 16x16 block, same
//           per-output semantics); a wave owns 32x32 outputs as 2x2 blocks.
//   valu  — the fma chains on the float64 vector ALU. A wave owns 16 rows x 64
//           columns; lane l keeps the chains of column l for the 16 rows. The
//           row operand reaches all lanes through a DPP row broadcast
//           (V_FMAC_F64 with row_newbcast:n takes src0 from lane n of each row of
//           16 lanes), so each lane loads one row value and one column value per
//           reduction index from LDS and issues 16 fmas.
// The Neumaier combine runs on the float64 vector ALU once per tile and output.
// All three stage 64x32 operand tiles in LDS as float64, laid out
// [reduction index][row or column], double buffered, with the next tile's
// global loads issued before the current tile's arithmetic.

#include <type_traits>

#include "common.hpp"

namespace detgemm {
namespace {

constexpr int KT = 32;        // the method's tile width along the reduction
constexpr int BM = 64;        // workgroup output rows
constexpr int BN = 64;        // workgroup output columns
constexpr int THREADS = 256;
constexpr int LS = 80;        // LDS row stride in doubles: 64 + 16 padding keeps the
                              // four reduction rows read by one wave in distinct bank halves

typedef double v4d __attribute__((ext_vector_type(4)));

// (s, c) <- Neumaier(s, c, p): s + p rounded, its exact error added to c.
__device__ inline void kbn_add(double& s, double& c, double p) {
  const double t = s + p;
  const double bp = t - s;
  const double ap = t - bp;
  const double e = (s - ap) + (p - bp);
  c = c + e;
  s = t;
}

// ---- operand staging --------------------------------------------------------
//
// One 64 x 32 slice (64 rows of A or columns of B, 32 reduction indices) per
// tile. Each thread moves 8 elements: x = t % 64 along the non-reduction dim,
// l = 8 * (t / 64) + j along the reduction. A reduction-contiguous source
// (element (x, l) at src[x * ld + l]) gives each thread 8 consecutive
// elements (one vector load); a reduction-major source (element (x, l) at
// src[l * ld + x]) gives the 64 lanes of a wave 64 consecutive elements per j.
// LDS layout: dst[l * LS + x], float64; a wave's 64 lanes write 64 consecutive
// doubles per store, so the stores are free of bank conflicts.

// Eight elements kept in registers as loaded until they are written to LDS, so
// that the vector-load and edge paths leave the same registers behind and the
// loads stay in flight across the arithmetic of the current tile. PACKED (a
// reduction-contiguous source, one vector load): 32-bit words as in memory.
// Otherwise one element per word (16-bit elements zero-extended): packing them
// right after eight separate loads would wait for those loads at once.
template <typename E, bool PACKED = true> struct alignas(16) Raw8 {
  static constexpr int NW = PACKED ? static_cast<int>(8 * sizeof(typename E::T) / 4) : 8;
  uint32_t w[NW];
};

template <typename T> __device__ inline uint32_t bits_of(T v);
template <> __device__ inline uint32_t bits_of<float>(float v) { return __float_as_uint(v); }
template <> __device__ inline uint32_t bits_of<uint16_t>(uint16_t v) { return v; }
template <> __device__ inline uint32_t bits_of<_Float16>(_Float16 v) { return __builtin_bit_cast(uint16_t, v); }

template <typename E> __device__ inline double up_bits(uint32_t b);
template <> __device__ inline double up_bits<F32>(uint32_t b) { return static_cast<double>(__uint_as_float(b)); }
template <> __device__ inline double up_bits<BF16>(uint32_t b) { return static_cast<double>(__uint_as_float(b << 16)); }
template <> __device__ inline double up_bits<F16>(uint32_t b) {
  return static_cast<double>(static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b))));
}

// Element j of a Raw8 as float64.
template <typename E, bool PACKED> __device__ inline double element(const Raw8<E, PACKED>& r, int j) {
  if constexpr (Raw8<E, PACKED>::NW == 8) return up_bits<E>(r.w[j]);
  return up_bits<E>((r.w[j >> 1] >> (16 * (j & 1))) & 0xffffu);
}

// XW (<= 64) is the slice's width along the non-reduction dimension; lanes
// past it repeat the last column's loads and fill LDS columns nobody reads.
template <typename E, bool RED_CONTIG, int XW = 64>
struct Stager {
  using T = typename E::T;
  static constexpr int64_t ES = sizeof(T);
  const T* __restrict__ src;
  const char* __restrict__ ubase;  // wave-uniform byte base of tile 0 (interior path)
  int64_t ustep;                   // bytes between consecutive tiles (uniform)
  int64_t uld;                     // bytes between reduction rows, reduction-major sources
  uint32_t voff;                   // this lane's byte offset from ubase (interior path)
  int64_t gx;                      // this thread's index along the non-reduction dim
  int64_t gl;                      // this thread's first reduction index in tile 0
  int64_t ld, xlen, llen;
  bool full;                       // interior path usable for this block (uniform)
  __amdgpu_buffer_rsrc_t rsrc;     // reduction-major interior path: the operand as a buffer
  uint32_t lane_off;               // reduction-major interior path: byte offset of the lane's column

  __device__ Stager(const T* src_, int64_t ld_, int64_t x0, int64_t xlen_, int64_t llen_, bool aligned, bool off32) {
    const int t = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    src = src_;
    ld = ld_;
    xlen = xlen_;
    llen = llen_;
    const int x = (t & 63) < XW ? (t & 63) : XW - 1;
    gx = x0 + x;
    gl = wave * 8;
    full = off32 && (x0 + XW <= xlen_) && (!RED_CONTIG || aligned);
    const char* b = reinterpret_cast<const char*>(src_);
    if (RED_CONTIG) {
      ubase = b + gl * ES;
      ustep = KT * ES;
      uld = 0;
      voff = static_cast<uint32_t>(gx * ld_ * ES);
    } else {
      ubase = b + (gl * ld_ + x0) * ES;
      ustep = KT * ld_ * ES;
      uld = ld_ * ES;
      voff = static_cast<uint32_t>(x * ES);
      // the buffer spans the operand (clamped to 31 bits: the interior path
      // only runs when every element offset fits, off32)
      const int64_t nbytes = ((llen_ - 1) * ld_ + xlen_) * ES;
      rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(src_), 0,
                                               static_cast<int>(nbytes < 0x7fffffff ? nbytes : 0x7fffffff), 0x00020000);
      lane_off = static_cast<uint32_t>(gx * ES);
    }
  }

  // Interior tiles (uniform test) load from a wave-uniform base plus a fixed
  // per-lane 32-bit offset, with no per-tile vector arithmetic (reduction-major
  // sources: buffer loads, the row offset in a scalar register); edge tiles load
  // every element from a clamped, always valid address and zero what lies
  // outside the operand. No lane-divergent branch, so the loads stay in flight.
  using Raw = Raw8<E, RED_CONTIG>;

  __device__ inline void load(int tile, Raw& r) const {
    const bool interior = full && static_cast<int64_t>(tile + 1) * KT <= llen;
    if (interior) {
      const char* tb = ubase + tile * ustep;
      if (RED_CONTIG) {
        r = *reinterpret_cast<const Raw*>(tb + voff);
        return;
      }
      // reduction-major: a per-lane column offset (vector) plus a per-row
      // offset (scalar), so the eight loads need no vector address arithmetic
      uint32_t e[8];
      const int row0 = static_cast<int>(static_cast<int64_t>(tile) * KT + gl);
      const int rstep = static_cast<int>(uld);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int soff = (row0 + j) * rstep;
        if constexpr (ES == 4)
          e[j] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, static_cast<int>(lane_off), soff, 0);
        else
          e[j] = __builtin_amdgcn_raw_buffer_load_b16(rsrc, static_cast<int>(lane_off), soff, 0);
      }
#pragma unroll
      for (int i = 0; i < Raw::NW; ++i)
        r.w[i] = (Raw::NW == 8) ? e[i] : (e[2 * i] | (e[2 * i + 1] << 16));
      return;
    }
    uint32_t e[8];
    const int64_t l0 = static_cast<int64_t>(tile) * KT + gl;
    const bool xok = gx < xlen;
    const int64_t xc = xok ? gx : xlen - 1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t l = l0 + j;
      const int64_t lc = l < llen ? l : llen - 1;
      const uint32_t v = bits_of<T>(RED_CONTIG ? src[xc * ld + lc] : src[lc * ld + xc]);
      e[j] = (xok && l < llen) ? v : 0u;
    }
#pragma unroll
    for (int i = 0; i < Raw::NW; ++i)
      r.w[i] = (Raw::NW == 8) ? e[i] : (e[2 * i] | (e[2 * i + 1] << 16));
  }

  __device__ inline void store(double* __restrict__ dst, const Raw& r) const {
    const int t = threadIdx.x;
    const int x = t & 63, l = (t >> 6) * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[(l + j) * LS + x] = element<E>(r, j);
  }
};

__device__ inline int tiles_of(int64_t red) { return static_cast<int>((red + KT - 1) / KT); }

// ---- valu kernel ------------------------------------------------------------

// acc = fma(a taken from lane N of this lane's row of 16, b, acc), one rounding.
template <int N> __device__ inline void fmac_bcast(double& acc, double a, double b) {
  asm("v_fmac_f64_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
      : "+v"(acc) : "v"(a), "v"(b), "i"(N));
}
template <int N> __device__ inline void fmac_rows(double (&p)[16], double a, double b) {
  fmac_bcast<N>(p[N], a, b);
  if constexpr (N + 1 < 16) fmac_rows<N + 1>(p, a, b);
}

template <typename E, bool A_RED_CONTIG, bool B_RED_CONTIG>
__global__ void __launch_bounds__(THREADS) exact_valu_kernel(GemmArgs args) {
  __shared__ double As[2][KT * LS];
  __shared__ double Bs[2][KT * LS];
  const int64_t tiles_n = (args.cols + BN - 1) / BN;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) / tiles_n) * BM;
  const int64_t col0 = (static_cast<int64_t>(blockIdx.x) % tiles_n) * BN;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wr = wave * 16;          // the wave's 16 rows inside the block

  const Stager<E, A_RED_CONTIG> sa(static_cast<const typename E::T*>(args.A), args.lda, row0, args.rows, args.red, args.vec_a, args.off32_a);
  const Stager<E, B_RED_CONTIG> sb(static_cast<const typename E::T*>(args.B), args.ldb, col0, args.cols, args.red, args.vec_b, args.off32_b);
  typename decltype(sa)::Raw ra;
  typename decltype(sb)::Raw rb;

  double s[16], c[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) { s[n] = 0.0; c[n] = 0.0; }

  const int ntiles = tiles_of(args.red);
  sa.load(0, ra);
  sb.load(0, rb);
  sa.store(As[0], ra);
  sb.store(Bs[0], rb);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = static_cast<int>(t & 1);
    const bool more = t + 1 < ntiles;
    if (more) { sa.load(t + 1, ra); sb.load(t + 1, rb); }
    const double* __restrict__ as = As[buf] + wr + (lane & 15);
    const double* __restrict__ bs = Bs[buf] + lane;
    double p[16];
#pragma unroll
    for (int n = 0; n < 16; ++n) p[n] = 0.0;
#pragma unroll 8
    for (int k = 0; k < KT; ++k) {
      const double a = as[k * LS];
      const double b = bs[k * LS];
      fmac_rows<0>(p, a, b);
    }
#pragma unroll
    for (int n = 0; n < 16; ++n) kbn_add(s[n], c[n], p[n]);
    if (more) { sa.store(As[buf ^ 1], ra); sb.store(Bs[buf ^ 1], rb); }
    __syncthreads();
  }

  typename E::T* __restrict__ Y = static_cast<typename E::T*>(args.out);
  const typename E::T* __restrict__ bias = static_cast<const typename E::T*>(args.bias);
  const int64_t col = col0 + lane;
  if (col < args.cols) {
    const double bj = bias ? E::up(bias[col]) : 0.0;
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const int64_t row = row0 + wr + n;
      if (row < args.rows) {
        double r = s[n] + c[n];
        if (bias) r = r + bj;
        Y[row * args.cols + col] = round_from_f64<E>(r);
      }
    }
  }
}

// ---- mfma4 kernel -----------------------------------------------------------
//
// V_MFMA_F64_4X4X4_4B_F64 operand layout (block g = 0..3, lane L):
//   A: L = 16k + 4g + i holds A_g[i][k];  B: L = 16k + 4g + j holds B_g[k][j];
//   D: L = 16i + 4g + j holds D_g[i][j].
// Wave w owns columns 16w .. 16w+15 of the 64-column block and all BMT rows
// (BMT = 64 or 48). Row fragment u (u < BMT / 16) puts row 16u + 4g + i in
// block g; column fragment r (r = 0..3) puts column 16w + 4((g + r) mod 4) + j
// in block g. Instruction (u, r) therefore covers rows 16u + 4g + i against
// columns 4((g + r) mod 4) + j for every block g, and the instructions cover
// the BMT x 16 outputs once. The 48-row form exists for launch balance: it
// turns grids such as 12 x 48 blocks of 64 x 64 (2.25 per compute unit) into
// 16 x 48 blocks of 48 x 64 (three per compute unit, all resident at once).

// O: the output type (E, or F32 for dW written as f32).
template <typename E, bool A_RED_CONTIG, bool B_RED_CONTIG, int NBUF, int BMT, typename O = E>
__global__ void __launch_bounds__(THREADS, NBUF == 1 ? 3 : 2) exact_mfma4_kernel(GemmArgs args) {
  // NBUF == 2: double-buffered LDS (80 KB), one barrier per tile, 2 workgroups per CU.
  // NBUF == 1: single LDS buffer (40 KB), two barriers per tile, 3 workgroups per CU.
  constexpr int NU = BMT / 16;
  static_assert(BMT % 16 == 0 && BMT <= BM, "row block");
  __shared__ double As[NBUF][KT * LS];
  __shared__ double Bs[NBUF][KT * LS];
  const int64_t tiles_n = (args.cols + BN - 1) / BN;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) / tiles_n) * BMT;
  const int64_t col0 = (static_cast<int64_t>(blockIdx.x) % tiles_n) * BN;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wn = wave * 16;
  const int lk = lane >> 4;           // k inside a group of four (operands); i (results)
  const int lg = (lane >> 2) & 3;     // block g
  const int le = lane & 3;            // i (A operand) / j (B operand, results)

  const Stager<E, A_RED_CONTIG, BMT> sa(static_cast<const typename E::T*>(args.A), args.lda, row0, args.rows, args.red, args.vec_a, args.off32_a);
  const Stager<E, B_RED_CONTIG> sb(static_cast<const typename E::T*>(args.B), args.ldb, col0, args.cols, args.red, args.vec_b, args.off32_b);
  typename decltype(sa)::Raw ra;
  typename decltype(sb)::Raw rb;

  int bcol[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) bcol[r] = wn + 4 * ((lg + r) & 3) + le;

  double s[NU][4], c[NU][4];
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) { s[u][r] = 0.0; c[u][r] = 0.0; }

  const int ntiles = tiles_of(args.red);
  sa.load(0, ra);
  sb.load(0, rb);
  sa.store(As[0], ra);
  sb.store(Bs[0], rb);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = NBUF == 2 ? (t & 1) : 0;
    const bool more = t + 1 < ntiles;
    if (more) { sa.load(t + 1, ra); sb.load(t + 1, rb); }
    const double* __restrict__ as = As[buf] + lk * LS + (lane & 15);
    const double* __restrict__ bs = Bs[buf] + lk * LS;
    double p[NU][4];
    double a[2][NU], b[2][4];
#pragma unroll
    for (int u = 0; u < NU; ++u) a[0][u] = as[16 * u];
#pragma unroll
    for (int r = 0; r < 4; ++r) b[0][r] = bs[bcol[r]];
#pragma unroll
    for (int g = 0; g < KT / 4; ++g) {
      const int cur = g & 1;
      if (g + 1 < KT / 4) {
        const int kr = (g + 1) * 4 * LS;
#pragma unroll
        for (int u = 0; u < NU; ++u) a[cur ^ 1][u] = as[kr + 16 * u];
#pragma unroll
        for (int r = 0; r < 4; ++r) b[cur ^ 1][r] = bs[kr + bcol[r]];
      }
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r)   // the chain of each tile starts from +0
          p[u][r] = __builtin_amdgcn_mfma_f64_4x4x4f64(a[cur][u], b[cur][r], g == 0 ? 0.0 : p[u][r], 0, 0, 0);
    }
    if (NBUF == 1) __syncthreads();   // every wave is done reading the single buffer
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) kbn_add(s[u][r], c[u][r], p[u][r]);
    if (more) { sa.store(As[NBUF == 2 ? buf ^ 1 : 0], ra); sb.store(Bs[NBUF == 2 ? buf ^ 1 : 0], rb); }
    __syncthreads();
  }

  typename O::T* __restrict__ Y = static_cast<typename O::T*>(args.out);
  const typename E::T* __restrict__ bias = static_cast<const typename E::T*>(args.bias);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t col = col0 + bcol[r];
    if (col >= args.cols) continue;
    const double bj = bias ? E::up(bias[col]) : 0.0;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int64_t row = row0 + 16 * u + 4 * lg + lk;   // result lane 16i + 4g + j
      if (row < args.rows) {
        double v = s[u][r] + c[u][r];
        if (bias) v = v + bj;
        Y[row * args.cols + col] = round_from_f64<O>(v);
      }
    }
  }
}

// ---- m16s kernel (default) ---------------------------------------------------
//
// The mfma4 kernel's structure (single LDS buffer, three workgroups per CU, 64
// or 48 rows x 64 columns, a wave owning all rows x 16 columns) with the
// tile's chains on V_MFMA_F64_16X16X4_F64: one instruction per 16-row block
// and k-step instead of four, and one B fragment read instead of four (the
// instruction computes each output as the same ascending fma chain over its
// four products, so the bits are unchanged). With 48-row blocks the running
// sums alternate between two register sets tile by tile (two tiles per loop
// trip), so Neumaier's s <- t costs no copy; with 64 rows that second set would
// not fit the registers three workgroups per CU leave.
template <typename E, bool A_RED_CONTIG, bool B_RED_CONTIG, int BMT, typename O = E>
__global__ void __launch_bounds__(THREADS, 3) exact_m16s_kernel(GemmArgs args) {
  constexpr int NU = BMT / 16;
  constexpr bool PP = NU <= 3;   // ping-pong running sums
  static_assert(BMT % 16 == 0 && BMT <= BM, "row block");
  __shared__ double As[KT * LS];
  __shared__ double Bs[KT * LS];
  const int64_t tiles_n = (args.cols + BN - 1) / BN;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) / tiles_n) * BMT;
  const int64_t col0 = (static_cast<int64_t>(blockIdx.x) % tiles_n) * BN;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wn = wave * 16;
  const int lr = lane & 15;   // row (A) / column (B, results) inside a 16 x 16 block
  const int lk = lane >> 4;   // k inside a group of four (operands); row group (results)
  const Stager<E, A_RED_CONTIG, BMT> sa(static_cast<const typename E::T*>(args.A), args.lda, row0, args.rows, args.red,
                                        args.vec_a, args.off32_a);
  const Stager<E, B_RED_CONTIG> sb(static_cast<const typename E::T*>(args.B), args.ldb, col0, args.cols, args.red,
                                   args.vec_b, args.off32_b);
  typename decltype(sa)::Raw ra;
  typename decltype(sb)::Raw rb;

  double s0[NU][4], s1[NU][4], c[NU][4];
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) { s0[u][e] = 0.0; s1[u][e] = 0.0; c[u][e] = 0.0; }

  const int ntiles = tiles_of(args.red);
  sa.load(0, ra);
  sb.load(0, rb);
  sa.store(As, ra);
  sb.store(Bs, rb);
  __syncthreads();

  // tile t: its chains, then (sout, c) <- Neumaier(sin, c, partial)
  auto step = [&](int t, double (&sin)[NU][4], double (&sout)[NU][4]) {
    const bool more = t + 1 < ntiles;
    if (more) { sa.load(t + 1, ra); sb.load(t + 1, rb); }
    const double* __restrict__ as = As + lk * LS + lr;
    const double* __restrict__ bs = Bs + lk * LS + wn + lr;
    v4d p[NU];
    double a[2][NU], b[2];
#pragma unroll
    for (int u = 0; u < NU; ++u) a[0][u] = as[16 * u];
    b[0] = bs[0];
#pragma unroll
    for (int g = 0; g < KT / 4; ++g) {
      const int cur = g & 1;
      if (g + 1 < KT / 4) {
        const int kr = (g + 1) * 4 * LS;
#pragma unroll
        for (int u = 0; u < NU; ++u) a[cur ^ 1][u] = as[kr + 16 * u];
        b[cur ^ 1] = bs[kr];
      }
#pragma unroll
      for (int u = 0; u < NU; ++u)   // the chain of each tile starts from +0
        p[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[cur][u], b[cur], g == 0 ? v4d{0.0, 0.0, 0.0, 0.0} : p[u], 0, 0,
                                                    0);
    }
    __syncthreads();   // every wave is done reading the single buffer
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {   // kbn_add with the new sum in a register of its own
        const double sv = sin[u][e], pv = p[u][e];
        const double tv = sv + pv;
        const double bp = tv - sv;
        const double ap = tv - bp;
        c[u][e] = c[u][e] + ((sv - ap) + (pv - bp));
        sout[u][e] = tv;
      }
    if (more) { sa.store(As, ra); sb.store(Bs, rb); }
    __syncthreads();
  };
  int t = 0;
  if constexpr (PP) {
    for (; t + 1 < ntiles; t += 2) {
      step(t, s0, s1);
      step(t + 1, s1, s0);
    }
  }
  for (; t < ntiles; ++t) {
    step(t, s0, s1);
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) s0[u][e] = s1[u][e];
  }

  typename O::T* __restrict__ Y = static_cast<typename O::T*>(args.out);
  const typename E::T* __restrict__ bias = static_cast<const typename E::T*>(args.bias);
  const int64_t col = col0 + wn + lr;
  if (col >= args.cols) return;
  const double bj = bias ? E::up(bias[col]) : 0.0;
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t row = row0 + 16 * u + 4 * e + lk;   // accumulator e of lane l: row 4e + l/16, column l%16
      if (row < args.rows) {
        double v = s0[u][e] + c[u][e];
        if (bias) v = v + bj;
        Y[row * args.cols + col] = round_from_f64<O>(v);
      }
    }
}

// ---- mfma16 kernel ----------------------------------------------------------

template <typename E, bool A_RED_CONTIG, bool B_RED_CONTIG>
__global__ void __launch_bounds__(THREADS) exact_mfma_kernel(GemmArgs args) {
  __shared__ double As[2][KT * LS];
  __shared__ double Bs[2][KT * LS];
  const int64_t tiles_n = (args.cols + BN - 1) / BN;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) / tiles_n) * BM;
  const int64_t col0 = (static_cast<int64_t>(blockIdx.x) % tiles_n) * BN;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wm = (wave >> 1) * 32;
  const int wn = (wave & 1) * 32;
  const int lr = lane & 15;   // row (A) / column (B, D) inside a 16x16 block
  const int lk = lane >> 4;   // k inside a group of four

  const Stager<E, A_RED_CONTIG> sa(static_cast<const typename E::T*>(args.A), args.lda, row0, args.rows, args.red, args.vec_a, args.off32_a);
  const Stager<E, B_RED_CONTIG> sb(static_cast<const typename E::T*>(args.B), args.ldb, col0, args.cols, args.red, args.vec_b, args.off32_b);
  typename decltype(sa)::Raw ra;
  typename decltype(sb)::Raw rb;

  double s[2][2][4], c[2][2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) { s[i][j][e] = 0.0; c[i][j][e] = 0.0; }

  const int ntiles = tiles_of(args.red);
  sa.load(0, ra);
  sb.load(0, rb);
  sa.store(As[0], ra);
  sb.store(Bs[0], rb);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = static_cast<int>(t & 1);
    const bool more = t + 1 < ntiles;
    if (more) { sa.load(t + 1, ra); sb.load(t + 1, rb); }
    const double* __restrict__ as = As[buf];
    const double* __restrict__ bs = Bs[buf];
    v4d p[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) p[i][j] = v4d{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int g = 0; g < KT / 4; ++g) {
      const int kr = 4 * g + lk;
      const double a0 = as[kr * LS + wm + lr];
      const double a1 = as[kr * LS + wm + 16 + lr];
      const double b0 = bs[kr * LS + wn + lr];
      const double b1 = bs[kr * LS + wn + 16 + lr];
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
        for (int e = 0; e < 4; ++e) kbn_add(s[i][j][e], c[i][j][e], p[i][j][e]);
    if (more) { sa.store(As[buf ^ 1], ra); sb.store(Bs[buf ^ 1], rb); }
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
        // accumulator e of lane l of a V_MFMA_F64_16X16X4 block is row 4e + l/16, column l%16
        const int64_t row = row0 + wm + 16 * i + 4 * e + lk;
        if (row < args.rows && col < args.cols) {
          double r = s[i][j][e] + c[i][j][e];
          if (bias) r = r + E::up(bias[col]);
          Y[row * args.cols + col] = round_from_f64<E>(r);
        }
      }
    }
}

// ---- skinny path -------------------------------------------------------------
//
// For few output rows (decode-sized batches) the blocked kernels leave most of
// the GPU idle: a handful of blocks each walk every tile in turn. The tile
// partials p_t of the different (row, column) outputs are independent of one
// another, and only the Neumaier combine is ordered, so this path computes
// all partials in parallel -- one wave per (tile, 64 columns), every row --
// into the stream's workspace, then combines them per output in tile order.
// The arithmetic is the definition above step for step, so the bits are those
// of the other kernels.
//   1. partials: P[t][row][col] = fma chain over the tile's indices from +0;
//      the wave upcasts its tile of A (rows x 32) into LDS once, and every
//      lane then reads those values as broadcasts;
//   2. combine: (s, c) <- Neumaier(s, c, P[t]) for t ascending; s + c, the
//      bias, one rounding.
constexpr int SK_ROWS = 32;   // row counts up to this take the skinny path (also the LDS row chunk)
constexpr int SK_ILP = 4;     // rows whose chains advance side by side

// One wave per (tile t, 64 columns): lane = column; the tile's 32 B values
// are loaded once, and SK_ILP rows' chains advance together.
template <typename E, bool A_RC, bool B_RC>
__global__ void __launch_bounds__(64) skinny_partial_kernel(const typename E::T* __restrict__ A, int64_t lda,
                                                            const typename E::T* __restrict__ B, int64_t ldb,
                                                            int64_t rows, int64_t cols, int64_t red, int64_t ncb,
                                                            double* __restrict__ P) {
  __shared__ double As[SK_ROWS * KT];
  const int lane = threadIdx.x;
  const int64_t t = blockIdx.x / ncb, cb = blockIdx.x - t * ncb;
  const int64_t c = cb * 64 + lane;
  const bool ok = c < cols;
  const int64_t cc = ok ? c : cols - 1;   // clamped column: loads stay inside B, nothing is stored
  const int64_t l0 = t * KT;
  const int cnt = static_cast<int>(red - l0 < KT ? red - l0 : KT);
  double b[KT];
#pragma unroll
  for (int j = 0; j < KT; ++j) {
    const int64_t l = l0 + (j < cnt ? j : cnt - 1);
    b[j] = E::up(B_RC ? B[cc * ldb + l] : B[l * ldb + cc]);
  }
  for (int64_t r0 = 0; r0 < rows; r0 += SK_ROWS) {
    const int nr = static_cast<int>(rows - r0 < SK_ROWS ? rows - r0 : SK_ROWS);
    __syncthreads();   // the previous chunk's reads are done (one wave: orders LDS only)
    // all of the chunk's loads are issued before any is used
    constexpr int PER = SK_ROWS * KT / 64;
    typename E::T av[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = lane + 64 * u;
      const int r = i / KT < nr ? i / KT : nr - 1, j = i % KT;
      const int64_t l = l0 + (j < cnt ? j : cnt - 1);
      av[u] = A_RC ? A[(r0 + r) * lda + l] : A[l * lda + r0 + r];
    }
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (lane + 64 * u < nr * KT) As[lane + 64 * u] = E::up(av[u]);
    __syncthreads();
    int r = 0;
    for (; r + SK_ILP <= nr; r += SK_ILP) {
      double p[SK_ILP];
#pragma unroll
      for (int q = 0; q < SK_ILP; ++q) p[q] = 0.0;
      if (cnt == KT) {
#pragma unroll
        for (int j = 0; j < KT; ++j)
#pragma unroll
          for (int q = 0; q < SK_ILP; ++q) p[q] = __builtin_fma(As[(r + q) * KT + j], b[j], p[q]);
      } else {
        for (int j = 0; j < cnt; ++j)
#pragma unroll
          for (int q = 0; q < SK_ILP; ++q) p[q] = __builtin_fma(As[(r + q) * KT + j], b[j], p[q]);
      }
      if (ok) {
#pragma unroll
        for (int q = 0; q < SK_ILP; ++q) P[(t * rows + r0 + r + q) * cols + c] = p[q];
      }
    }
    for (; r < nr; ++r) {
      double p = 0.0;
      if (cnt == KT) {
#pragma unroll
        for (int j = 0; j < KT; ++j) p = __builtin_fma(As[r * KT + j], b[j], p);
      } else {
        for (int j = 0; j < cnt; ++j) p = __builtin_fma(As[r * KT + j], b[j], p);
      }
      if (ok) P[(t * rows + r0 + r) * cols + c] = p;
    }
  }
}

template <typename E, typename O>
__global__ void __launch_bounds__(256) skinny_combine_kernel(const double* __restrict__ P, int64_t T, int64_t rows,
                                                             int64_t cols, const typename E::T* __restrict__ bias,
                                                             typename O::T* __restrict__ Y) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // row * cols + col
  if (i >= rows * cols) return;
  const int64_t stride = rows * cols;
  double s = 0.0, c = 0.0;
  int64_t t = 0;
  for (; t + 32 <= T; t += 32) {   // 32 partials in flight at a time
    double v[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = P[(t + j) * stride + i];
#pragma unroll
    for (int j = 0; j < 32; ++j) kbn_add(s, c, v[j]);
  }
  if (t < T) {   // the rest (fewer than 32) likewise, loads first
    double v[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = t + j < T ? P[(t + j) * stride + i] : 0.0;
#pragma unroll
    for (int j = 0; j < 32; ++j)
      if (t + j < T) kbn_add(s, c, v[j]);
  }
  double v = s + c;
  if (bias) v = v + E::up(bias[i % cols]);
  Y[i] = round_from_f64<O>(v);
}

template <typename E, bool AC, bool BC, typename O>
hipError_t launch_skinny(const GemmArgs& a, hipStream_t stream) {
  const int64_t T = (a.red + KT - 1) / KT;
  const int64_t ncb = (a.cols + 63) / 64;
  const int64_t n_p = T * a.rows * a.cols;
  if (T * ncb > 0x7fffffff || (a.rows * a.cols + 255) / 256 > 0x7fffffff) return hipErrorInvalidConfiguration;
  void* ws = nullptr;
  hipError_t e = stream_workspace(stream, sizeof(double) * static_cast<size_t>(n_p), &ws);
  if (e != hipSuccess) return e;
  double* P = static_cast<double*>(ws);
  using T_ = typename E::T;
  hipLaunchKernelGGL((skinny_partial_kernel<E, AC, BC>), dim3(static_cast<unsigned>(T * ncb)), dim3(64), 0, stream,
                     static_cast<const T_*>(a.A), a.lda, static_cast<const T_*>(a.B), a.ldb, a.rows, a.cols, a.red,
                     ncb, P);
  hipLaunchKernelGGL((skinny_combine_kernel<E, O>), dim3(static_cast<unsigned>((a.rows * a.cols + 255) / 256)),
                     dim3(256), 0, stream, P, T, a.rows, a.cols, static_cast<const T_*>(a.bias),
                     static_cast<typename O::T*>(a.out));
  return hipGetLastError();
}

// ---- launch -----------------------------------------------------------------

// Launch balance of the default kernel: every block of one grid does the same
// work, proportional to its rows, and blocks are spread evenly over the
// compute units (up to three resident on each). The time of a grid follows
// the rows of the busiest compute unit, ceil(blocks / units) x (rows per
// block); take 48-row blocks when that is smaller (measured: GPT-2 c_fc dW
// 48-row 850 us against 64-row 1110 us; QKV dW, where 64-row blocks leave at
// most two per unit, 844 against 787 us). Both forms give identical bits.
bool use_48_rows(const GemmArgs& a) {
  const int64_t units = a.num_cu > 0 ? a.num_cu : 1;
  const int64_t tn = (a.cols + BN - 1) / BN;
  const int64_t l64 = (tn * ((a.rows + 63) / 64) + units - 1) / units * 64;
  const int64_t l48 = (tn * ((a.rows + 47) / 48) + units - 1) / units * 48;
  return l48 < l64;
}

// Small grids over short reductions: with at most two 64 x 64 blocks per
// compute unit (and 48-row blocks no better) and at most 4096 reduction
// indices, the mfma16 kernel's double-buffered stage runs them a little faster
// than the default (measured: fwd of 512 rows into 3072 columns 74.8 -> 73.3
// us, dX of 1024 rows 165.8 -> 161.8); over long reductions the default is
// faster (GPT-2 QKV dW 731 -> 699 us). Same bits.
bool use_mfma16(const GemmArgs& a) {
  const int64_t units = a.num_cu > 0 ? a.num_cu : 1;
  return ((a.cols + BN - 1) / BN) * ((a.rows + BM - 1) / BM) <= 2 * units && a.red <= 4096;
}

// The few-rows path keeps every tile partial: 8 * rows * cols * ceil(red / 32)
// bytes. It is taken automatically only up to this size (a dW with few output
// rows has a reduction over the batch, whose tile count has no bound), and the
// blocked kernels, which need no workspace and give the same bits, run when
// the workspace cannot be had.
constexpr int64_t SK_MAX_BYTES = int64_t(64) << 20;

bool use_skinny(const GemmArgs& a) {
  if (a.rows > SK_ROWS) return false;
  const int64_t T = (a.red + KT - 1) / KT;
  return T <= SK_MAX_BYTES / 8 / (a.rows * a.cols);   // 8 T rows cols <= SK_MAX_BYTES without overflow
}

template <typename E, bool AC, bool BC, typename O = E>
hipError_t launch_typed(const GemmArgs& a, int variant, hipStream_t stream) {
  const bool automatic = variant < 0;
  if (automatic) variant = use_skinny(a) ? 5 : use_48_rows(a) ? 4 : use_mfma16(a) ? 1 : 0;
  if (variant == 5) {
    const hipError_t e = launch_skinny<E, AC, BC, O>(a, stream);
    if (!(automatic && e == hipErrorOutOfMemory)) return e;
    (void)hipGetLastError();   // nothing was enqueued: the blocked kernels below, same bits
    variant = use_48_rows(a) ? 4 : use_mfma16(a) ? 1 : 0;
  }
  // f32 output: the default kernel in its two row-block forms, or the mfma4
  // kernel in the same two forms (identical bits)
  if constexpr (!std::is_same<O, E>::value) {
    if (variant != 4 && variant != 6 && variant != 7) variant = 0;
  }
  const int64_t blocks = ((a.cols + BN - 1) / BN) * ((a.rows + BM - 1) / BM);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
  // (variants 1 .. 3 write the input type only; for f32 output variant is 0, 4, 6 or 7 here)
  const int64_t b48 = ((a.cols + BN - 1) / BN) * ((a.rows + 47) / 48);
  if (b48 > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (variant == 1)
    hipLaunchKernelGGL((exact_mfma_kernel<E, AC, BC>), grid, dim3(THREADS), 0, stream, a);
  else if (variant == 2)
    hipLaunchKernelGGL((exact_valu_kernel<E, AC, BC>), grid, dim3(THREADS), 0, stream, a);
  else if (variant == 3)
    hipLaunchKernelGGL((exact_mfma4_kernel<E, AC, BC, 2, 64>), grid, dim3(THREADS), 0, stream, a);
  else if (variant == 4)
    hipLaunchKernelGGL((exact_m16s_kernel<E, AC, BC, 48, O>), dim3(static_cast<unsigned>(b48)), dim3(THREADS), 0,
                       stream, a);
  else if (variant == 6)
    hipLaunchKernelGGL((exact_mfma4_kernel<E, AC, BC, 1, 64, O>), grid, dim3(THREADS), 0, stream, a);
  else if (variant == 7)
    hipLaunchKernelGGL((exact_mfma4_kernel<E, AC, BC, 1, 48, O>), dim3(static_cast<unsigned>(b48)), dim3(THREADS), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((exact_m16s_kernel<E, AC, BC, 64, O>), grid, dim3(THREADS), 0, stream, a);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_op(Op op, const GemmArgs& a, int variant, hipStream_t stream) {
  switch (op) {
    case OP_FWD: return launch_typed<E, true, false>(a, variant, stream);   // X[i][k], W[k][j]
    case OP_DX:  return launch_typed<E, true, true>(a, variant, stream);    // dY[i][n], W[q][n]
    case OP_DW:   // X[i][q], dY[i][j]
      if (a.out_f32) return launch_typed<E, false, false, F32>(a, variant, stream);
      return launch_typed<E, false, false>(a, variant, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_exact(Op op, Dt dt, const GemmArgs& a, int variant, hipStream_t stream) {
  switch (dt) {
    case DT_F32: return launch_op<F32>(op, a, variant, stream);
    case DT_BF16: return launch_op<BF16>(op, a, variant, stream);
    case DT_F16: return launch_op<F16>(op, a, variant, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace detgemm
