// Fast tier: matrix-core GEMM with f32 accumulation over a fixed walk of the
// reduction (sgemm-bi 0.1.2 PyPI page, "Determinism contracts": tensor-core
// tier with f32 accumulate, bit-identical across runs, forward batch-invariant
// across all M, two tile families with identical bits, shape-only dispatch).
//
// Determinism and batch invariance
//   * Every output element is produced by the same matrix-core instruction
//     (V_MFMA_F32_32X32X16_BF16 / _F16 for 16-bit inputs, V_MFMA_F32_16X16X4_F32
//     for f32 inputs), stepping through the reduction from index 0 upward in
//     steps of the instruction's depth, starting from a zero accumulator. No
//     split of the reduction, no atomics. The bias is then added in f32 and the
//     sum rounded once to the output type.
//   * An output element's arithmetic therefore involves only its own row of A,
//     its own column of B and the reduction length: not the row count, the tile
//     family or the position of its tile. Padding rows and reduction indices
//     are zeros, which add nothing.
//   * The tile families -- for f32 inputs the staged 128x128 kernel and the
//     plain 64x64 one here; for 16-bit inputs the tile shapes of fast16w.hip
//     and fast16.hip -- differ only in how outputs are grouped into
//     workgroups and how operands reach the matrix cores.

#include "common.hpp"
#include "transpose.hpp"

namespace detgemm {
namespace {

constexpr int THREADS = 256;  // 4 waves, 2x2
constexpr int KS = 32;        // reduction depth staged in LDS per step

typedef float v4f __attribute__((ext_vector_type(4)));

template <typename E> struct Mfma;

// 16x16 outputs per instruction, depth 4; lane l holds A[l%16][l/16],
// B[l/16][l%16]; accumulator i of lane l is D[4*(l/16)+i][l%16].
template <> struct Mfma<F32> {
  static constexpr int BLK = 16, DEPTH = 4, PER = 1, ACC = 4;
  using Acc = v4f;
  __device__ static inline Acc step(const float* a, const float* b, Acc c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(*a, *b, c, 0, 0, 0);
  }
  __device__ static inline int row(int lane, int i) { return 4 * (lane / 16) + i; }
};

// Stage a KS-deep slice of an operand into LDS, layout dst[x][l] (reduction
// contiguous, row stride LD) for x < X (row of A or column of B), l < KS.
//   red_contig: element (x, l) is src[(x0 + x) * ld + l0 + l]
//   otherwise : element (x, l) is src[(l0 + l) * ld + x0 + x]
// Out-of-range elements are zeros. Global reads follow the contiguous index.
template <typename T, int X, int LD, bool RED_CONTIG>
__device__ inline void stage(T* __restrict__ dst, const T* __restrict__ src, int64_t ld,
                             int64_t x0, int64_t xlen, int64_t l0, int64_t llen) {
  for (int idx = threadIdx.x; idx < X * KS; idx += THREADS) {
    int x, l;
    if (RED_CONTIG) { x = idx / KS; l = idx % KS; }
    else            { l = idx / X;  x = idx % X; }
    const int64_t gx = x0 + x, gl = l0 + l;
    T v = T(0);
    if (gx < xlen && gl < llen) v = RED_CONTIG ? src[gx * ld + gl] : src[gl * ld + gx];
    dst[x * LD + l] = v;
  }
}

template <typename E, int BM, int BN, bool A_RED_CONTIG, bool B_RED_CONTIG>
__global__ void __launch_bounds__(THREADS) fast_kernel(GemmArgs args) {
  using T = typename E::T;
  using M = Mfma<E>;
  constexpr int LD = KS + 16 / (int)sizeof(T) * 2;   // padded row stride (keeps 16-byte alignment)
  constexpr int WM = BM / 2, WN = BN / 2;            // per-wave outputs
  constexpr int NI = WM / M::BLK, NJ = WN / M::BLK;  // blocks per wave
  __shared__ __attribute__((aligned(16))) T As[BM * LD];
  __shared__ __attribute__((aligned(16))) T Bs[BN * LD];

  const T* __restrict__ A = static_cast<const T*>(args.A);
  const T* __restrict__ B = static_cast<const T*>(args.B);
  const int64_t tiles_n = (args.cols + BN - 1) / BN;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) / tiles_n) * BM;
  const int64_t col0 = (static_cast<int64_t>(blockIdx.x) % tiles_n) * BN;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wm = (wave >> 1) * WM;
  const int wn = (wave & 1) * WN;
  const int lx = lane % M::BLK;                 // row of A / column of B in a block
  const int lk = (lane / M::BLK) * M::PER;      // first reduction index of the lane

  typename M::Acc acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < M::ACC; ++e) acc[i][j][e] = 0.0f;

  for (int64_t l0 = 0; l0 < args.red; l0 += KS) {
    stage<T, BM, LD, A_RED_CONTIG>(As, A, args.lda, row0, args.rows, l0, args.red);
    stage<T, BN, LD, B_RED_CONTIG>(Bs, B, args.ldb, col0, args.cols, l0, args.red);
    __syncthreads();
#pragma unroll
    for (int d = 0; d < KS; d += M::DEPTH) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = M::step(&As[(wm + i * M::BLK + lx) * LD + d + lk], &Bs[(wn + j * M::BLK + lx) * LD + d + lk], acc[i][j]);
    }
    __syncthreads();
  }

  T* __restrict__ Y = static_cast<T*>(args.out);
  const T* __restrict__ bias = static_cast<const T*>(args.bias);
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t col = col0 + wn + j * M::BLK + lx;
#pragma unroll
      for (int e = 0; e < M::ACC; ++e) {
        const int64_t row = row0 + wm + i * M::BLK + M::row(lane, e);
        if (row < args.rows && col < args.cols) {
          float r = acc[i][j][e];
          if (bias) r = r + E::to_f32(bias[col]);
          Y[row * args.cols + col] = round_from_f32<E>(r);
        }
      }
    }
}

template <typename E, int BM, int BN, bool AC, bool BC>
hipError_t launch_typed(const GemmArgs& a, hipStream_t stream) {
  const int64_t blocks = ((a.cols + BN - 1) / BN) * ((a.rows + BM - 1) / BM);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fast_kernel<E, BM, BN, AC, BC>), dim3(static_cast<unsigned>(blocks)), dim3(THREADS), 0, stream, a);
  return hipGetLastError();
}

template <typename E, int BM, int BN>
hipError_t launch_op(Op op, const GemmArgs& a, hipStream_t stream) {
  switch (op) {
    case OP_FWD: return launch_typed<E, BM, BN, true, false>(a, stream);
    case OP_DX:  return launch_typed<E, BM, BN, true, true>(a, stream);
    case OP_DW:  return launch_typed<E, BM, BN, false, false>(a, stream);
  }
  return hipErrorInvalidValue;
}

// f32 inputs, large tiles: the same instruction sequence per output as
// fast_kernel (V_MFMA_F32_16X16X4_F32 over 4-index steps from index 0, from a
// zero accumulator; bias in f32; one rounding), staged for speed: 128 x 128
// outputs per workgroup, 32 reduction indices per stage, both operands kept in
// LDS as [l][x] (row stride 144 floats: the four reduction rows one fragment
// read touches fall 16 banks apart), double buffered, the next stage's global
// loads (16 bytes where the operand allows) in registers during the current
// stage's matrix work, one barrier per stage.
constexpr int F32_BM = 128, F32_LDX = F32_BM + 16;

// Four consecutive elements along the operand's contiguous dimension starting
// at (x, l) -- along l when RC, along x otherwise -- zero outside the operand.
template <bool RC>
__device__ inline void load4_f32(const float* __restrict__ src, int64_t ld, int64_t x, int64_t l, int64_t xlen,
                                 int64_t llen, bool vec, float (&v)[4]) {
  const int64_t first = RC ? l : x, lim = RC ? llen : xlen;
  const bool in = RC ? (x < xlen) : (l < llen);
  const float* p = RC ? src + x * ld + l : src + l * ld + x;
  if (in && vec && first + 4 <= lim) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = (in && first + e < lim) ? p[e] : 0.0f;
}

template <bool A_RC, bool B_RC>
__global__ void __launch_bounds__(THREADS) fast_f32_kernel(GemmArgs args) {
  constexpr int BM = F32_BM, BN = F32_BM, LDX = F32_LDX;
  constexpr int NI = 4, NJ = 4;                 // 16 x 16 blocks per wave (64 x 64 outputs)
  constexpr int Q = BM * KS / 4 / THREADS;      // float4 pieces per thread per operand and stage
  __shared__ __attribute__((aligned(16))) float As[2][KS * LDX];
  __shared__ __attribute__((aligned(16))) float Bs[2][KS * LDX];
  const float* __restrict__ A = static_cast<const float*>(args.A);
  const float* __restrict__ B = static_cast<const float*>(args.B);
  const int64_t tiles_n = (args.cols + BN - 1) / BN;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) / tiles_n) * BM;
  const int64_t col0 = (static_cast<int64_t>(blockIdx.x) % tiles_n) * BN;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int lx = lane & 15, lk = lane >> 4;
  const bool va = args.vec_a, vb = args.vec_b;

  // piece q of this thread: RC -- x = idx % 128, l = 4 (idx / 128); otherwise
  // l = idx / 32, x = 4 (idx % 32) (idx = t + 256 q), so that consecutive
  // lanes write consecutive LDS addresses.
  float ra[Q][4], rb[Q][4];
  auto load = [&](int64_t l0) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int idx = t + THREADS * q;
      const int xa = A_RC ? idx % BM : 4 * (idx % (BM / 4)), la = A_RC ? 4 * (idx / BM) : idx / (BM / 4);
      const int xb = B_RC ? idx % BN : 4 * (idx % (BN / 4)), lb = B_RC ? 4 * (idx / BN) : idx / (BN / 4);
      load4_f32<A_RC>(A, args.lda, row0 + xa, l0 + la, args.rows, args.red, va, ra[q]);
      load4_f32<B_RC>(B, args.ldb, col0 + xb, l0 + lb, args.cols, args.red, vb, rb[q]);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int idx = t + THREADS * q;
      if (A_RC) {
        const int x = idx % BM, l = 4 * (idx / BM);
#pragma unroll
        for (int e = 0; e < 4; ++e) As[buf][(l + e) * LDX + x] = ra[q][e];
      } else {
        const int x = 4 * (idx % (BM / 4)), l = idx / (BM / 4);
        *reinterpret_cast<float4*>(&As[buf][l * LDX + x]) = make_float4(ra[q][0], ra[q][1], ra[q][2], ra[q][3]);
      }
      if (B_RC) {
        const int x = idx % BN, l = 4 * (idx / BN);
#pragma unroll
        for (int e = 0; e < 4; ++e) Bs[buf][(l + e) * LDX + x] = rb[q][e];
      } else {
        const int x = 4 * (idx % (BN / 4)), l = idx / (BN / 4);
        *reinterpret_cast<float4*>(&Bs[buf][l * LDX + x]) = make_float4(rb[q][0], rb[q][1], rb[q][2], rb[q][3]);
      }
    }
  };

  v4f acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0f;

  const int64_t nst = (args.red + KS - 1) / KS;
  load(0);
  store(0);
  __syncthreads();
  for (int64_t st = 0; st < nst; ++st) {
    const int buf = static_cast<int>(st & 1);
    const bool more = st + 1 < nst;
    if (more) load((st + 1) * KS);
    const float* as = As[buf];
    const float* bs = Bs[buf];
#pragma unroll
    for (int d = 0; d < KS; d += 4) {
      float a[NI], b[NJ];
#pragma unroll
      for (int i = 0; i < NI; ++i) a[i] = as[(d + lk) * LDX + wm + 16 * i + lx];
#pragma unroll
      for (int j = 0; j < NJ; ++j) b[j] = bs[(d + lk) * LDX + wn + 16 * j + lx];
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) store(buf ^ 1);
    __syncthreads();
  }

  float* __restrict__ Y = static_cast<float*>(args.out);
  const float* __restrict__ bias = static_cast<const float*>(args.bias);
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t col = col0 + wn + 16 * j + lx;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = row0 + wm + 16 * i + 4 * lk + e;
        if (row < args.rows && col < args.cols) {
          float r = acc[i][j][e];
          if (bias) r = r + bias[col];
          Y[row * args.cols + col] = r;
        }
      }
    }
}

template <bool AC, bool BC>
hipError_t launch_f32_large(const GemmArgs& a, hipStream_t stream) {
  const int64_t blocks = ((a.cols + F32_BM - 1) / F32_BM) * ((a.rows + F32_BM - 1) / F32_BM);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fast_f32_kernel<AC, BC>), dim3(static_cast<unsigned>(blocks)), dim3(THREADS), 0, stream, a);
  return hipGetLastError();
}

// f32 inputs: family 0 is the staged 128 x 128 kernel, family 1 the plain
// 64 x 64 one (the same instruction sequence per output, so the same bits).
hipError_t launch_family_f32(Op op, int family, const GemmArgs& a, hipStream_t stream) {
  if (family == 0) {
    switch (op) {
      case OP_FWD: return launch_f32_large<true, false>(a, stream);
      case OP_DX:  return launch_f32_large<true, true>(a, stream);
      case OP_DW:  return launch_f32_large<false, false>(a, stream);
    }
    return hipErrorInvalidValue;
  }
  return launch_op<F32, 64, 64>(op, a, stream);
}

}  // namespace

// First family choice from the output width and the reduction length (the
// families give identical bits, so this only affects speed; launch_fast
// refines family 0 with the row count). f32: the staged 128 x 128 kernel
// unless the output is narrow or the reduction short, where the 64 x 64 tiles
// of the plain kernel keep more of the chip busy. 16-bit: the large
// direct-to-LDS tiles for outputs of 256 columns or more and for dW, the small
// register-staged tiles otherwise.
int fast_auto_family(Op op, Dt dt, int64_t cols, int64_t red) {
  if (dt == DT_F32) return (cols >= 512 && red >= 512) ? 0 : 1;
  (void)red;
  return (op == OP_DW || cols >= 256) ? 0 : 1;
}

// dW of 16-bit inputs has few output tiles when K x N is small, so its
// reduction over M is split into S chunks of whole 64-row stages, each
// accumulated from 0 in f32 and combined in ascending chunk order. S follows
// from the shape alone -- a reference tiling of 256 x 192 outputs and a
// notional 256 compute units, never the device -- so every kernel and every
// device gives the same bits; chunks are at least 8 stages long.
int fast_dw_split(int64_t m, int64_t k, int64_t n, int* chunk_stages) {
  const int64_t nst = (m + 63) / 64;
  const int64_t tiles = ((k + 255) / 256) * ((n + 191) / 192);
  int64_t s = tiles < 128 ? 256 / tiles : 1;
  if (s > 16) s = 16;
  if (s > nst / 8) s = nst / 8;
  if (s < 1) s = 1;
  const int64_t c = (nst + s - 1) / s;
  *chunk_stages = static_cast<int>(c);
  return static_cast<int>((nst + c - 1) / c);
}

hipError_t launch_fast16_w_dw_bt(Dt dt, const GemmArgs& a, int shape, hipStream_t stream);   // fast16w.hip

hipError_t launch_fast(Op op, Dt dt, const GemmArgs& a, int family, hipStream_t stream) {
  // family < 0: automatic (a forced family runs its own kernels, so that the
  // tests can compare every family on every shape)
  const bool automatic = family < 0;
  if (automatic) family = fast_auto_family(op, dt, a.cols, a.red);
  if (op == OP_DW && dt != DT_F32 && a.partial == nullptr) {
    int chunk = 0;
    const int split = fast_dw_split(a.red, a.rows, a.cols, &chunk);
    // Fewer than 128 workgroups of 256 x 192 tiles (chunks included): the small
    // register-staged tiles keep more compute units busy (measured: 2048 x
    // 1024 x 1024 dW 29.7 -> 17.6 us, 4096 x 256 x 512 26.9 -> 13.0 us).
    if (family == 0 && ((a.rows + 255) / 256) * ((a.cols + 191) / 192) * split < 128) family = 1;
    // The default family may take the smaller operand (x or dY, both
    // reduction-major) copied transposed: the kernel then stages that one
    // straight into LDS, as the forward's x, and only the other through
    // registers. Tile shape and copy by measured speed: without a split, four
    // fat waves (128 x 96 each) with the copy; split into long chunks, eight
    // waves (64 x 96 each) with the copy; split into short chunks (at most 20
    // stages), four fat waves without it. Same values in the same instruction
    // order in every form, so the same bits.
    const bool base = family == 0 && a.red % 64 == 0 && a.red <= int64_t(64) * 65535;
    const bool tr0 = base && a.rows <= a.cols && a.vec_b && a.off32_b && a.rows * a.red * 2 < (int64_t(1) << 31);
    const bool trb0 = base && !tr0 && a.vec_a && a.off32_a && a.cols * a.red * 2 < (int64_t(1) << 31);
    const bool copy = (tr0 || trb0) && (split == 1 || chunk > 20);
    const bool tr = copy && tr0, trb = copy && trb0;
    const int shape = split > 1 && copy ? 0 : 5;
    if (split > 1 || copy) {
      // chunk partials (when split) and the transposed copy in the stream's
      // workspace; with a split, the ordered combine writes the output
      const size_t count = static_cast<size_t>(a.rows) * static_cast<size_t>(a.cols);
      const size_t pbytes = split > 1 ? (count * sizeof(float) * static_cast<size_t>(split) + 255) / 256 * 256 : 0;
      const size_t tbytes = tr ? static_cast<size_t>(a.rows) * static_cast<size_t>(a.red) * 2
                          : trb ? static_cast<size_t>(a.cols) * static_cast<size_t>(a.red) * 2 : 0;
      void* ws = nullptr;
      hipError_t e = stream_workspace(stream, pbytes + tbytes, &ws);
      if (e != hipSuccess) return e;
      GemmArgs p = a;
      p.partial = split > 1 ? static_cast<float*>(ws) : nullptr;
      p.split = split;
      p.chunk_stages = chunk;
      if (tr) {
        uint16_t* xt = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + pbytes);
        e = launch_transpose<uint16_t>(a.A, a.red, a.rows, xt, stream);
        if (e != hipSuccess) return e;
        p.A = xt;
        p.lda = a.red;
        p.vec_a = true;
        p.off32_a = true;
        p.a_bytes = static_cast<int64_t>(tbytes);
        e = launch_fast16_w(OP_FWD, dt, p, shape, stream);   // x rows now contiguous along the reduction
      } else if (trb) {
        uint16_t* yt = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + pbytes);
        e = launch_transpose<uint16_t>(a.B, a.red, a.cols, yt, stream);
        if (e != hipSuccess) return e;
        p.B = yt;
        p.ldb = a.red;
        p.vec_b = true;
        p.off32_b = true;
        p.b_bytes = static_cast<int64_t>(tbytes);
        e = launch_fast16_w_dw_bt(dt, p, shape, stream);   // dY columns now contiguous along the reduction
      } else {
        e = launch_fast(op, dt, p, family == 0 ? 15 : family, stream);
      }
      if (e != hipSuccess) return e;
      if (split == 1) return hipSuccess;
      return launch_combine(dt, a.out_f32, p.partial, split, static_cast<int64_t>(count), a.out, stream);
    }
    if (family == 0) family = 15;   // no split, no copy: four fat waves
  }
  // Forward of 16-bit inputs with at most 32 rows (decode-sized batches): the
  // work is a stream of the weight, which the tiled kernels read through a
  // handful of tiles; the few-rows kernel gives every 32 output columns a
  // workgroup of its own. Same instruction sequence per output, so the same
  // bits. Family 16 forces it (where it applies).
  if (op == OP_FWD && dt != DT_F32 && (automatic || family == 16) && fast16_skinny_ok(a))
    return launch_fast16_skinny(dt, a, stream);
  if (family == 16) family = 0;
  // Forward of 16-bit inputs with many rows and a long reduction or a wide
  // output: the weight copied transposed first ([n][k], contiguous along the
  // reduction), so that the kernel stages both operands straight into LDS, as
  // for dX. Same values in the same instruction order, so the same bits.
  // Measured: GPT-2 c_proj (k = 3072) 53.9 -> 49.8 us and 4096 x 11008 x 4096
  // 915 -> 849 us at m = 8192; with k = 768: QKV (n = 2304) 46.8 -> 44.6 us,
  // c_fc (n = 3072) 50.7 -> 50.1 us and at m = 16384 97.7 -> 90.1 us,
  // 4096 x 1024 x 4096 56.3 -> 52.1 us; slower into 768 columns
  // (attention projection 18.0 -> 19.5 us) and, the copy being 2 k n bytes
  // each way, on few rows.
  if (op == OP_FWD && dt != DT_F32 && family == 0 && fast16_w_ok(a) && a.rows >= 4096 &&
      (a.red >= 3072 || a.cols >= 1536) &&
      a.red % 8 == 0 && a.cols % 8 == 0 && a.red <= int64_t(64) * 65535 && a.cols * a.red * 2 < (int64_t(1) << 31)) {
    void* ws = nullptr;
    hipError_t e = stream_workspace(stream, static_cast<size_t>(a.cols) * static_cast<size_t>(a.red) * 2, &ws);
    if (e == hipErrorOutOfMemory) {
      (void)hipGetLastError();   // no room for the copy: the plain form below, same bits
    } else {
      if (e != hipSuccess) return e;
      e = launch_transpose<uint16_t>(a.B, a.red, a.cols, ws, stream);
      if (e != hipSuccess) return e;
      GemmArgs p = a;
      p.B = ws;
      p.ldb = a.red;
      p.vec_b = true;
      p.off32_b = true;
      p.b_bytes = a.cols * a.red * 2;
      return launch_fast16_w(OP_DX, dt, p, fast16_w_shape(a.cols, a.red), stream);   // both operands along rows
    }
  }
  switch (dt) {
    case DT_F32: return launch_family_f32(op, family == 1 ? 1 : 0, a, stream);
    case DT_BF16:
    case DT_F16:
      // family 0: eight-wave large tiles where the shape allows it (10 + s:
      // a given tile shape s of that kernel); otherwise, and family 1, the
      // four-wave register-staged kernel. Identical bits.
      if (family == 0 && fast16_w_ok(a)) {
        const int sh = op == OP_DW ? 0 : fast16_w_shape(a.cols, a.red);
        // Automatic choice, fewer tiles than compute units and rows that fill
        // the smaller tiles exactly (ragged ones measured slower: m = 200,
        // 27.9 against 19.9 us): smaller tiles for speed, the same bits -- fwd on fast16's
        // 128 x 64 tiles, dX on 64 x 192 tiles two per compute unit
        // (measured at m = 256 .. 2048: fwd 768 -> 3072 at m = 256 20.2 ->
        // 10.0 us, at m = 128 19.5 -> 9.7 us, dX into 768 columns at m = 1024
        // 34.1 -> 26.7 us; from m = 1 to 64 the large tiles stay faster,
        // 19.2 against 22 - 27 us).
        const int64_t bm = sh == 0 ? 256 : 128;
        if (automatic && op != OP_DW && a.rows % (op == OP_FWD ? 128 : 64) == 0 &&
            ((a.rows + bm - 1) / bm) * ((a.cols + 191) / 192) < 256)
          return op == OP_FWD ? launch_fast16(op, dt, a, 1, stream) : launch_fast16_w(op, dt, a, 3, stream);
        return launch_fast16_w(op, dt, a, sh, stream);
      }
      if (family >= 10 && fast16_w_ok(a)) return launch_fast16_w(op, dt, a, family - 10, stream);
      return launch_fast16(op, dt, a, family == 1 ? 1 : 0, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace detgemm
