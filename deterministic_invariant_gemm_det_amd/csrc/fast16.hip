// Fast tier for 16-bit inputs (bf16, f16): V_MFMA_F32_32X32X16_{BF16,F16}
// with f32 accumulation over a fixed ascending walk of the reduction.
//
// Contract (sgemm-bi 0.1.2 PyPI page, "Determinism contracts", tensor-core
// tier): bit-identical across runs, forward batch-invariant across all M, two
// tile families with identical bits, shape-only dispatch.
//
// Every output element is the result of the same sequence of instructions:
// acc = 0, then acc = MFMA(acc, A[row, 16s .. 16s+15], B[16s .. 16s+15, col])
// for s = 0, 1, ... in order, then acc + bias rounded once to the output type.
// Nothing in that sequence depends on the row count, the tile family or the
// tile's position: padding rows/columns and reduction indices past the end are
// zeros. The families differ only in how outputs are grouped into workgroups.
//
// Workgroup: 256 threads = 4 waves in 2 x 2. Family 0 computes 256 x 128
// outputs per workgroup (a wave owns 128 x 64 = 4 x 2 blocks of 32 x 32),
// family 1 computes 128 x 64 (a wave owns 64 x 32 = 2 x 1 blocks). Each stage
// covers 64 reduction indices. Operands are copied to LDS in their memory
// order: a source whose reduction index is contiguous is kept [row][k] and a
// lane reads its 8-element fragment with one 16-byte LDS load; a source whose
// reduction index is the row index (the weight of the forward, both operands of
// dW) is kept [k][row] and a lane gathers its fragment with two gfx950
// transposing LDS reads (DS_READ_B64_TR_B16: within each group of 16 lanes,
// lane i receives element i % 4 of the 8-byte pieces read by lanes
// i / 4 + 4q, q = 0..3, i.e. four consecutive reduction indices of one column).
// The next stage's global loads are issued before the current stage's
// matrix-core work.

#include "common.hpp"

namespace detgemm {
namespace {

constexpr int THREADS = 256;
constexpr int BK = 64;            // reduction indices per LDS stage
constexpr int LDK = BK + 8;       // LDS row stride in elements (16-byte padding)

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

template <typename E> __device__ inline v16f mfma_step(v4u a, v4u b, v16f c);
template <> __device__ inline v16f mfma_step<BF16>(v4u a, v4u b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}
template <> __device__ inline v16f mfma_step<F16>(v4u a, v4u b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
}

template <typename T> __device__ inline uint16_t raw16(T v) { return __builtin_bit_cast(uint16_t, v); }

// Staging of one operand slice: X rows (of A) or columns (of B) by BK reduction
// indices. Each thread copies 16-byte vectors along the contiguous dimension.
//   RED_CONTIG: element (x, l) at src[x * ld + l]; LDS dst[x * LDK + l].
//   otherwise : element (x, l) at src[l * ld + x]; LDS dst[l * LDX + x] with
//               LDX = X + 32, so that the four rows a transposing read touches
//               fall in different LDS banks.
template <typename E, int X, bool RED_CONTIG>
struct Stage {
  using T = typename E::T;
  static constexpr int NV = X * BK / (8 * THREADS);   // 16-byte vectors per thread
  static constexpr int LDX = X + 32;
  static constexpr int LDS_ELEMS = RED_CONTIG ? X * LDK : BK * LDX;
  static constexpr int VPR = RED_CONTIG ? BK / 8 : X / 8;   // vectors per LDS row
  static constexpr int RPV = THREADS / VPR;                  // LDS rows between a thread's vectors
  static_assert(NV >= 1 && (X * BK) % (8 * THREADS) == 0 && THREADS % VPR == 0, "unsupported tile");
  v4u v[NV];
  __amdgpu_buffer_rsrc_t rsrc;   // the whole operand
  uint32_t voff;                 // byte offset of this thread's vector 0 in stage 0
  uint32_t vstep;                // bytes between a thread's consecutive vectors
  uint32_t sstep;                // bytes between consecutive stages

  // Vector i of thread t: idx = t + i * THREADS; LDS row idx / VPR, 8-wide piece idx % VPR.
  __device__ inline void init(const T* src, int64_t ld, int64_t x0, int64_t bytes) {
    const int t = threadIdx.x;
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(src), 0, static_cast<int>(bytes < 0x7fffffff ? bytes : 0x7fffffff), 0x00020000);
    const int r = t / VPR, c = 8 * (t % VPR);
    if (RED_CONTIG) {
      voff = static_cast<uint32_t>(((x0 + r) * ld + c) * 2);
      vstep = static_cast<uint32_t>(RPV * ld * 2);
      sstep = BK * 2;
    } else {
      voff = static_cast<uint32_t>((r * ld + x0 + c) * 2);
      vstep = static_cast<uint32_t>(RPV * ld * 2);
      sstep = static_cast<uint32_t>(BK * ld * 2);
    }
  }

  // Interior stage: one buffer load per vector from a per-thread offset plus a
  // uniform one; nothing per stage is computed on the vector ALU.
  __device__ inline void load_fast(int st) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, st * sstep + i * vstep, 0);
  }

  // Edge stage: element-wise loads from clamped, always valid addresses,
  // zeros outside the operand.
  __device__ inline void load_edge(const T* __restrict__ src, int64_t ld, int64_t x0, int64_t xlen,
                                   int64_t l0, int64_t llen) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = t + i * THREADS;
      const int r = idx / VPR, c = 8 * (idx % VPR);
      const int64_t gx = RED_CONTIG ? x0 + r : x0 + c;   // first x of the vector
      const int64_t gl = RED_CONTIG ? l0 + c : l0 + r;   // first l of the vector
      uint16_t e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t x = RED_CONTIG ? gx : gx + j;
        const int64_t l = RED_CONTIG ? gl + j : gl;
        const bool ok = x < xlen && l < llen;
        const int64_t xc = x < xlen ? x : xlen - 1;
        const int64_t lc = l < llen ? l : llen - 1;
        const uint16_t val = raw16(RED_CONTIG ? src[xc * ld + lc] : src[lc * ld + xc]);
        e[j] = ok ? val : uint16_t(0);
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) v[i][w] = static_cast<uint32_t>(e[2 * w]) | (static_cast<uint32_t>(e[2 * w + 1]) << 16);
    }
  }

  __device__ inline void store(T* __restrict__ dst) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = t + i * THREADS;
      const int r = idx / VPR, c = 8 * (idx % VPR);
      *reinterpret_cast<v4u*>(dst + r * (RED_CONTIG ? LDK : LDX) + c) = v[i];
    }
  }

  // The lane's 8-element fragment of the 32-wide block starting at xb, for the
  // reduction step starting at d: elements (xb + lane % 32, d + 8 * (lane / 32) + j).
  __device__ inline v4u frag(const T* __restrict__ S, int xb, int d) const {
    const int lane = threadIdx.x & 63;
    if (RED_CONTIG) {
      return *reinterpret_cast<const v4u*>(&S[(xb + (lane & 31)) * LDK + d + 8 * (lane >> 5)]);
    } else {
      typedef short v4s __attribute__((ext_vector_type(4)));
      const int g = lane >> 4, L = lane & 15;
      const int x = xb + 16 * (g & 1) + 4 * (L & 3);
      const int k = d + 8 * (g >> 1) + (L >> 2);
      const T* p0 = &S[k * LDX + x];
      const T* p1 = &S[(k + 4) * LDX + x];
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p0));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p1));
      typedef uint32_t v2u __attribute__((ext_vector_type(2)));
      const v2u a = __builtin_bit_cast(v2u, lo), b = __builtin_bit_cast(v2u, hi);
      return v4u{a[0], a[1], b[0], b[1]};
    }
  }
};

template <typename E, int BM, int BN, bool A_RED_CONTIG, bool B_RED_CONTIG>
__global__ void __launch_bounds__(THREADS, 2) fast16_kernel(GemmArgs args) {
  using T = typename E::T;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int NI = WM / 32, NJ = WN / 32;
  using SA = Stage<E, BM, A_RED_CONTIG>;
  using SB = Stage<E, BN, B_RED_CONTIG>;
  __shared__ __attribute__((aligned(16))) T As[SA::LDS_ELEMS];
  __shared__ __attribute__((aligned(16))) T Bs[SB::LDS_ELEMS];

  const T* __restrict__ A = static_cast<const T*>(args.A);
  const T* __restrict__ B = static_cast<const T*>(args.B);
  const int64_t tiles_n = (args.cols + BN - 1) / BN;
  const int64_t ntiles = tiles_n * ((args.rows + BM - 1) / BM);
  // for a split reduction, block b is tile b mod ntiles of chunk b / ntiles
  int64_t tb = blockIdx.x;
  int chunk = 0;
  if (args.partial) {
    chunk = static_cast<int>(tb / ntiles);
    tb -= chunk * ntiles;
  }
  const int64_t row0 = (tb / tiles_n) * BM;
  const int64_t col0 = (tb % tiles_n) * BN;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wm = (wave >> 1) * WM;
  const int wn = (wave & 1) * WN;
  const int lx = lane & 31;          // column of a result block

  const bool rows_full = row0 + BM <= args.rows;
  const bool cols_full = col0 + BN <= args.cols;

  SA sa;
  SB sb;
  sa.init(A, args.lda, row0, args.a_bytes);
  sb.init(B, args.ldb, col0, args.b_bytes);
  const bool fast_a = args.vec_a && args.off32_a && rows_full;
  const bool fast_b = args.vec_b && args.off32_b && cols_full;

  v16f acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // stages s0 .. nst - 1 (all of them, or one chunk of a split reduction)
  const int nst_all = static_cast<int>((args.red + BK - 1) / BK);
  const int s0 = args.partial ? chunk * args.chunk_stages : 0;
  const int nst = args.partial ? (nst_all - s0 < args.chunk_stages ? nst_all : s0 + args.chunk_stages) : nst_all;
  {
    const int64_t l0 = static_cast<int64_t>(s0) * BK;
    const bool kfull = l0 + BK <= args.red;
    if (fast_a && kfull) sa.load_fast(s0); else sa.load_edge(A, args.lda, row0, args.rows, l0, args.red);
    if (fast_b && kfull) sb.load_fast(s0); else sb.load_edge(B, args.ldb, col0, args.cols, l0, args.red);
  }
  for (int st = s0; st < nst; ++st) {
    sa.store(As);
    sb.store(Bs);
    __syncthreads();
    if (st + 1 < nst) {
      const int64_t l0 = static_cast<int64_t>(st + 1) * BK;
      const bool kfull = l0 + BK <= args.red;
      if (fast_a && kfull) sa.load_fast(st + 1); else sa.load_edge(A, args.lda, row0, args.rows, l0, args.red);
      if (fast_b && kfull) sb.load_fast(st + 1); else sb.load_edge(B, args.ldb, col0, args.cols, l0, args.red);
    }
#pragma unroll
    for (int d = 0; d < BK; d += 16) {
      v4u af[NI], bf[NJ];
#pragma unroll
      for (int i = 0; i < NI; ++i) af[i] = sa.frag(As, wm + 32 * i, d);
#pragma unroll
      for (int j = 0; j < NJ; ++j) bf[j] = sb.frag(Bs, wn + 32 * j, d);
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma_step<E>(af[i], bf[j], acc[i][j]);
    }
    __syncthreads();
  }

  const bool interior = rows_full && cols_full;
  if (args.partial || args.out_f32) {
    // split reduction: this chunk's f32 partials; f32 output: the accumulators
    // themselves (no bias in dW)
    float* __restrict__ P = args.partial ? args.partial + static_cast<int64_t>(chunk) * args.rows * args.cols
                                         : static_cast<float*>(args.out);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t col = col0 + wn + 32 * j + lx;
      if (!interior && col >= args.cols) continue;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int64_t rb = row0 + wm + 32 * i + 4 * (lane >> 5);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int rr = 8 * (e / 4) + (e % 4);
          if (interior || rb + rr < args.rows) P[(rb + rr) * args.cols + col] = acc[i][j][e];
        }
      }
    }
    return;
  }
  T* __restrict__ Y = static_cast<T*>(args.out);
  const T* __restrict__ bias = static_cast<const T*>(args.bias);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int64_t col = col0 + wn + 32 * j + lx;
    if (!interior && col >= args.cols) continue;
    const float bj = bias ? E::to_f32(bias[col]) : 0.0f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      // accumulator e of lane l is row 8*(e/4) + 4*(l/32) + e%4 of the block
      T* yb = Y + (row0 + wm + 32 * i + 4 * (lane >> 5)) * args.cols + col;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rr = 8 * (e / 4) + (e % 4);
        if (interior || row0 + wm + 32 * i + 4 * (lane >> 5) + rr < args.rows) {
          float r = acc[i][j][e];
          if (bias) r = r + bj;
          yb[rr * args.cols] = round_from_f32<E>(r);
        }
      }
    }
  }
}

template <typename E, int BM, int BN, bool AC, bool BC>
hipError_t launch_typed(const GemmArgs& a, hipStream_t stream) {
  const int64_t blocks = ((a.cols + BN - 1) / BN) * ((a.rows + BM - 1) / BM) * (a.partial ? a.split : 1);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fast16_kernel<E, BM, BN, AC, BC>), dim3(static_cast<unsigned>(blocks)), dim3(THREADS), 0, stream, a);
  return hipGetLastError();
}

template <typename E, int BM, int BN>
hipError_t launch_op(Op op, const GemmArgs& a, hipStream_t stream) {
  switch (op) {
    case OP_FWD: return launch_typed<E, BM, BN, true, false>(a, stream);   // X[i][k], W[k][j]
    case OP_DX:  return launch_typed<E, BM, BN, true, true>(a, stream);    // dY[i][n], W[q][n]
    case OP_DW:  return launch_typed<E, BM, BN, false, false>(a, stream);  // X[i][q], dY[i][j]
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fast16(Op op, Dt dt, const GemmArgs& a, int family, hipStream_t stream) {
  if (dt == DT_BF16)
    return family == 0 ? launch_op<BF16, 256, 128>(op, a, stream) : launch_op<BF16, 128, 64>(op, a, stream);
  if (dt == DT_F16)
    return family == 0 ? launch_op<F16, 256, 128>(op, a, stream) : launch_op<F16, 128, 64>(op, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace detgemm
