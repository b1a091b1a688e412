// Fast tier, forward with few rows (m <= 32), 16-bit inputs.
//
// Same arithmetic as the tiled kernels, hence the same bits for every output
// element (sgemm-bi 0.1.2 PyPI page, "Determinism contracts": bit-identical
// and batch-invariant across M): acc = 0, then acc =
// V_MFMA_F32_32X32X16_{BF16,F16}(x[row, 16s .. 16s+15], w[16s .. 16s+15, col],
// acc) for s = 0 .. 4 ceil(k / 64) - 1 in order (indices past k are zeros,
// as in the tiled kernels' stages of 64), then acc + bias rounded once.
//
// With few rows the work is a stream of the weight: all m rows fit one 32-row
// matrix block, so each 32 columns of output are one chain of dependent
// matrix instructions, and the time goes to reading w. One workgroup of nine
// waves owns 32 columns. Waves 1 .. 8 move the weight's 128-row chunks
// ([k][32], 64-byte rows) and the x rows below m of the matching 32 x 128
// piece through registers (plain 16-byte loads, D chunks in flight per wave)
// into a ring of R LDS slots; wave 0 runs the chain one chunk behind its
// reads: while the matrix instructions of chunk c - 1 run, it reads chunk c's
// x fragments (16-byte LDS loads) and weight fragments (two transposing loads,
// DS_READ_B64_TR_B16, per instruction). One barrier per chunk publishes it
// and hands back the slot read before it.
//
// Direct-to-LDS loads are not used here: streamed from beyond the L2 by one
// workgroup per compute unit they reached about half the rate of register
// loads (a strip-streaming probe on gfx950: ~30 against ~57 GB/s per CU).
//
// Applicability (checked on the host): k a multiple of 8, both operands and
// their rows 16-byte aligned, every byte offset below 2^31. x rows >= m and
// weight rows >= k lie outside their buffers and read as zeros; x pieces at
// or past k are redirected outside the buffer; weight columns >= n only reach
// outputs that are never stored.

#include "common.hpp"

namespace detgemm {
namespace sk {

constexpr int CK = 128;                 // reduction indices per chunk (8 steps of 16)
constexpr int W_BYTES = CK * 32 * 2;    // weight chunk: 128 rows x 32 columns, 64-byte rows
constexpr int X_BYTES = 32 * CK * 2;    // x chunk: 32 rows x 128 indices, 256-byte rows
constexpr int SLOT = W_BYTES + X_BYTES;
constexpr int R = 4;                    // LDS ring slots
constexpr int D = 6;                    // chunks each loader wave holds in flight in registers
constexpr int LOADERS = 8;              // waves 1 .. LOADERS move the operands; wave 0 runs the chain
constexpr int BPW = 8 / LOADERS;        // 1 KB blocks of each chunk (weight, and x) per loader wave
constexpr int THREADS = 64 * (LOADERS + 1);
constexpr uint32_t OUTSIDE = 0x80000000u;   // a byte offset past every buffer this path takes

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

template <typename E> __device__ inline v16f mfma_step(v4u a, v4u b, v16f c);
template <> __device__ inline v16f mfma_step<BF16>(v4u a, v4u b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}
template <> __device__ inline v16f mfma_step<F16>(v4u a, v4u b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
}

// s_waitcnt: no LDS operation outstanding (vector-memory count left free).
constexpr int WAIT_LGKM0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);

// x chunk layout: row r (256 bytes) holds the chunk's 128 indices as 16
// pieces of 16 bytes, piece p in slot p XOR f(r), f(r) = (r XOR r / 8) mod 16,
// so that the 32 rows of one fragment read spread over the banks.
__host__ __device__ constexpr int xf(int r) { return (r ^ (r >> 3)) & 15; }
__host__ __device__ constexpr int xoff(int r, int p) { return r * 256 + 16 * (p ^ xf(r)); }

// One chunk's fragments for the chain: x (A operand; lane l: row l mod 32,
// indices 16 s + 8 (l / 32) .. + 7) and the weight (B operand; two transposing
// reads per step: rows 16 s + 8 (g / 2) + L / 4 and + 4, columns 16 (g mod 2)
// + 4 (L mod 4), g = l / 16, L = l mod 16). All 8 steps are read even for a
// last chunk of 4: the reads stay inside the slot and the extra ones go unused.
__device__ inline void read_chunk(v4u (&fa)[8], v4u (&fb)[8], const char* slot, int xrow, int xpiece, int wfrag) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    fa[s] = *reinterpret_cast<const v4u*>(slot + W_BYTES + xoff(xrow, 2 * s + xpiece));
    const char* wp = slot + s * 16 * 64 + wfrag;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(wp));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(wp + 4 * 64));
    const v2u bl = __builtin_bit_cast(v2u, lo), bh = __builtin_bit_cast(v2u, hi);
    fb[s] = v4u{bl[0], bl[1], bh[0], bh[1]};
  }
}

template <typename E, int N>
__device__ inline void run_chain(v16f& acc, const v4u (&fa)[8], const v4u (&fb)[8]) {
#pragma unroll
  for (int s = 0; s < N; ++s) acc = mfma_step<E>(fa[s], fb[s], acc);
}

// The next chunk's 24 LDS reads are placed 3 after each matrix instruction of
// the current chain, so that they issue while each instruction waits for the
// previous one's result.
__device__ inline void interleave_reads() {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one matrix instruction
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // three LDS reads
  }
}

// wave 0's side of barrier c: its reads of chunk c - 1 are complete (so the
// loaders may refill that slot after the barrier), and chunk c is in LDS after it
__device__ inline void sync_chunk() {
  __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

template <typename E>
__global__ void __launch_bounds__(THREADS, 1) skinny_fwd_kernel(GemmArgs a) {
  using T = typename E::T;
  __shared__ __attribute__((aligned(1024))) char lds[R * SLOT];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t col0 = static_cast<int64_t>(blockIdx.x) * 32;
  const int64_t K = a.red, N = a.cols, M = a.rows;
  const int nsteps = static_cast<int>(4 * ((K + 63) / 64));   // the tiled kernels' step count
  const int nch = (nsteps + 7) / 8;

  if (wave != 0) {
    // loader wave w, blocks gi = BPW (w - 1) + q, q < BPW of each chunk:
    // weight rows 16 gi + lane / 4, columns 8 (lane mod 4) .. + 7, to LDS byte
    // 1024 gi + 16 lane; x row 4 gi + lane / 16, piece (lane mod 16) XOR f(row),
    // to x byte 1024 gi + 16 lane. x rows >= m are never loaded: their LDS
    // bytes are cleared once and stay zero.
    const auto wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.B), 0, static_cast<int>(a.b_bytes), 0x00020000);
    const auto xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.A), 0, static_cast<int>(a.a_bytes), 0x00020000);
    uint32_t w_off[BPW], x_off[BPW], x_k[BPW];
    bool x_live[BPW];
    int lds_at[BPW];
    for (int q = 0; q < BPW; ++q) {
      const int gi = BPW * (wave - 1) + q;
      w_off[q] = static_cast<uint32_t>(((16 * gi + (lane >> 2)) * N + col0 + 8 * (lane & 3)) * 2);
      const int xrow = 4 * gi + (lane >> 4);
      const int p = (lane & 15) ^ xf(xrow);
      x_live[q] = xrow < M;
      x_k[q] = static_cast<uint32_t>(8 * p);
      x_off[q] = static_cast<uint32_t>((xrow * K + 8 * p) * 2);
      lds_at[q] = 1024 * gi + 16 * lane;
    }
    for (int sl = 0; sl < R; ++sl)
      for (int q = 0; q < BPW; ++q)
        if (!x_live[q]) *reinterpret_cast<v4u*>(lds + sl * SLOT + W_BYTES + lds_at[q]) = v4u{0, 0, 0, 0};
    v4u wv[D][BPW], xv[D][BPW];
    // loads are unconditional (dead x lanes and chunks past the end read from
    // outside the buffers), so that the counts the compiler waits on stay exact
    auto load = [&](int c, v4u (&w)[BPW], v4u (&x)[BPW]) {
      const uint32_t k0 = static_cast<uint32_t>(c * CK);
      const bool in = c < nch;
#pragma unroll
      for (int q = 0; q < BPW; ++q) {
        w[q] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(
            wr, in ? w_off[q] + k0 * static_cast<uint32_t>(N) * 2u : OUTSIDE, 0, 0));
        x[q] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(
            xr, in && x_live[q] && k0 + x_k[q] < static_cast<uint32_t>(K) ? x_off[q] + 2u * k0 : OUTSIDE, 0, 0));
      }
    };
    // chunk c to its slot (free: wave 0 finished reading chunk c - R before
    // barrier c - R + 1), the registers refilled with chunk c + D, then barrier c
    auto put = [&](int c, v4u (&w)[BPW], v4u (&x)[BPW]) {
      char* slot = lds + (c % R) * SLOT;
#pragma unroll
      for (int q = 0; q < BPW; ++q) {
        *reinterpret_cast<v4u*>(slot + lds_at[q]) = w[q];
        if (x_live[q]) *reinterpret_cast<v4u*>(slot + W_BYTES + lds_at[q]) = x[q];
      }
      load(c + D, w, x);
      __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
      __asm__ volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();   // chunk c is in LDS
      __asm__ volatile("" ::: "memory");
    };
#pragma unroll
    for (int j = 0; j < D; ++j) load(j, wv[j], xv[j]);
    int c = 0;
    for (; c + D <= nch; c += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) put(c + j, wv[j], xv[j]);
    }
#pragma unroll
    for (int j = 0; j < D - 1; ++j)
      if (c + j < nch) put(c + j, wv[j], xv[j]);
    return;
  }

  v16f acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
  const int g = lane >> 4, L = lane & 15;
  const int wfrag = ((8 * (g >> 1) + (L >> 2)) * 32 + 16 * (g & 1) + 4 * (L & 3)) * 2;
  const int xrow = lane & 31, xpiece = lane >> 5;
  auto slot = [&](int c) { return lds + (c % R) * SLOT; };
  // one chunk ahead: chunk c's fragments are read while chunk c - 1's matrix
  // instructions run; every chunk but the last has 8 steps
  const bool last_full = nsteps % 8 == 0;
  v4u a0[8], b0[8], a1[8], b1[8];
  sync_chunk();
  read_chunk(a0, b0, slot(0), xrow, xpiece, wfrag);
  int c = 1;
  for (; c + 1 < nch; c += 2) {
    sync_chunk();
    read_chunk(a1, b1, slot(c), xrow, xpiece, wfrag);
    run_chain<E, 8>(acc, a0, b0);
    interleave_reads();
    sync_chunk();
    read_chunk(a0, b0, slot(c + 1), xrow, xpiece, wfrag);
    run_chain<E, 8>(acc, a1, b1);
    interleave_reads();
  }
  if (c == nch - 1) {
    sync_chunk();
    read_chunk(a1, b1, slot(c), xrow, xpiece, wfrag);
    run_chain<E, 8>(acc, a0, b0);
    interleave_reads();
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
    if (last_full) run_chain<E, 8>(acc, a1, b1);
    else run_chain<E, 4>(acc, a1, b1);
  } else {
    if (last_full) run_chain<E, 8>(acc, a0, b0);
    else run_chain<E, 4>(acc, a0, b0);
  }

  // acc[e] of lane l is output (8 (e / 4) + 4 (l / 32) + e mod 4, l mod 32)
  const int64_t col = col0 + (lane & 31);
  if (col >= N) return;
  T* __restrict__ Y = static_cast<T*>(a.out);
  const T* __restrict__ bias = static_cast<const T*>(a.bias);
  const float b = bias ? E::to_f32(bias[col]) : 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int64_t row = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
    if (row < M) {
      float r = acc[e];
      if (bias) r = r + b;
      Y[row * N + col] = round_from_f32<E>(r);
    }
  }
}

template <typename E>
hipError_t launch_typed(const GemmArgs& a, hipStream_t stream) {
  const int64_t blocks = (a.cols + 31) / 32;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((skinny_fwd_kernel<E>), dim3(static_cast<unsigned>(blocks)), dim3(THREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sk

// The few-rows forward applies: m <= 32; k a multiple of 8; operands and rows
// 16-byte aligned; every byte offset the kernel forms below 2^31 (x: 32 rows
// of k; the weight: k + 128 rows of n, the last chunk's rows past k).
constexpr int64_t CKH = sk::CK;
bool fast16_skinny_ok(const GemmArgs& a) {
  return a.rows <= 32 && a.red % 8 == 0 && a.vec_a && a.vec_b && a.off32_a && a.off32_b &&
         a.a_bytes < (int64_t(1) << 31) && a.b_bytes < (int64_t(1) << 31) && a.red * 64 < (int64_t(1) << 31) &&
         (a.red + CKH) * a.cols * 2 < (int64_t(1) << 31) && a.lda == a.red && a.ldb == a.cols;
}

hipError_t launch_fast16_skinny(Dt dt, const GemmArgs& a, hipStream_t stream) {
  if (!fast16_skinny_ok(a)) return hipErrorInvalidValue;
  if (dt == DT_BF16) return sk::launch_typed<BF16>(a, stream);
  if (dt == DT_F16) return sk::launch_typed<F16>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace detgemm
