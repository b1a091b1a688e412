// Fast tier, 16-bit inputs, large tiles fed by direct-to-LDS loads.
//
// Same arithmetic as fast16.hip (and therefore the same bits for every output
// element): acc = 0, then acc = V_MFMA_F32_32X32X16_{BF16,F16}(acc, A[row,
// 16s .. 16s+15], B[16s .. 16s+15, col]) for s = 0, 1, ... in order, then
// acc + bias rounded once (sgemm-bi 0.1.2 PyPI page, "Determinism contracts").
// Only the way operands reach the matrix cores differs.
//
// Workgroup: 256 threads = 4 waves in 2 x 2, 256 x 128 outputs, a wave owns
// 128 x 64 (4 x 2 blocks of 32 x 32, 128 accumulator registers). Each stage
// covers 64 reduction indices and is copied from global memory straight into
// LDS with buffer loads that write LDS (each wave instruction fills 1 KB of LDS,
// lane l at byte 16 l). Three LDS stages form a ring: stage s + 2 is requested
// while stage s is being multiplied, and one barrier per stage both publishes
// stage s and frees the buffer of stage s - 1.
//
// LDS layouts (no padding; a 16-byte XOR swizzle keeps reads free of bank
// conflicts):
//   reduction-contiguous operand: [row][64 k], 128 bytes per row; 16-byte piece
//     c of row r is stored at piece c ^ (r mod 8). A lane reads its 8-element
//     fragment with one 16-byte LDS load.
//   reduction-major operand (the forward weight, both operands of dW):
//     [k][X columns]; 16-byte piece j of row k is stored at piece
//     j ^ 4 (k mod 4). A lane gathers its fragment with two transposing reads
//     (DS_READ_B64_TR_B16).
//
// Applicability (checked on the host): the reduction length is a multiple of
// 64, operands are 16-byte aligned with 16-byte aligned rows, and every byte
// offset fits in 31 bits. Rows or columns past the end of an operand are read
// as zeros (buffer range check) or as neighbouring data that only reaches
// outputs that are never stored.

#include "common.hpp"

namespace detgemm {
namespace dl {

constexpr int THREADS = 256;
constexpr int BM = 256, BN = 128, BK = 64, NSTAGE = 3;
constexpr int WM = BM / 2, WN = BN / 2, NI = WM / 32, NJ = WN / 32;
constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4s lds_v4s;

template <typename E> __device__ inline v16f mfma_step(v4u a, v4u b, v16f c);
template <> __device__ inline v16f mfma_step<BF16>(v4u a, v4u b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}
template <> __device__ inline v16f mfma_step<F16>(v4u a, v4u b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
}

// s_waitcnt immediate (gfx9 encoding): at most `vm` vector-memory operations
// outstanding, no LDS operation outstanding, exports unconstrained.
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | (7 << 4) | (0 << 8) | (((vm >> 4) & 3) << 14); }

// One operand: X rows (A) or columns (B) by BK reduction indices per stage.
template <int X, bool RC>
struct Operand {
  static constexpr int NQ = X * BK * 2 / 1024 / 4;   // 1 KB wave instructions per wave per stage
  static constexpr int LPR = X / 8;                   // KM: lanes per LDS row (16-byte pieces per row)
  static constexpr int RPI = 64 / LPR;                // KM: LDS rows per instruction
  v4u rsrc;              // buffer resource (uniform)
  uint32_t voff[NQ];     // per-lane source byte offset of instruction q in stage 0
  uint32_t sstep;        // source bytes between stages

  __device__ inline void init(const void* src, int64_t ld, int64_t x0, int64_t bytes) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // buffer resource: base address, stride 0, size in bytes (reads past it
    // return zeros), 32-bit data format
    const uint64_t base = reinterpret_cast<uint64_t>(src);
    rsrc = v4u{static_cast<uint32_t>(base), static_cast<uint32_t>(base >> 32) & 0xffffu,
               static_cast<uint32_t>(bytes), 0x00020000u};
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int g = wave * NQ + q;   // instruction index within the stage
      if (RC) {
        const int r = 8 * g + (lane >> 3), c = (lane & 7) ^ (r & 7);
        voff[q] = static_cast<uint32_t>(((x0 + r) * ld + 8 * c) * 2);
      } else {
        const int k = RPI * g + lane / LPR, j = (lane % LPR) ^ (4 * (k & 3));
        voff[q] = static_cast<uint32_t>((k * ld + x0 + 8 * j) * 2);
      }
    }
    sstep = static_cast<uint32_t>(RC ? BK * 2 : BK * ld * 2);
  }

  // Request stage st into the LDS block at `dst` (1 KB per wave instruction).
  // The loads are written as inline assembly: the compiler then does not
  // track them as LDS writes and does not drain them before every LDS read of
  // another ring slot. Completion is waited for explicitly (vmcnt) before the
  // barrier that publishes a stage. M0 holds the LDS address of the
  // instruction's 1 KB block; one wait state separates its write from the load.
  // The whole byte offset travels in the VGPR operand (scalar offset 0), so
  // the buffer's range check sees all of it: a 16-byte piece past the end of
  // the operand reads zeros instead of memory beyond the allocation.
  __device__ inline void issue(char* dst, int st) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)dst));
    const uint32_t soff = static_cast<uint32_t>(st) * sstep;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const uint32_t m0 = lds + 1024u * static_cast<uint32_t>(wave * NQ + q);
      const uint32_t off = voff[q] + soff;
      __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                       :
                       : "s"(m0), "v"(off), "s"(rsrc)
                       : "memory", "m0");
    }
  }

  // The lane's fragment of the 32-wide block at xb for reduction step d:
  // elements (xb + lane % 32, d + 8 * (lane / 32) + j), j = 0..7, from the
  // operand block at `base` in LDS.
  __device__ inline v4u frag(const char* base, int xb, int d) const {
    const int lane = threadIdx.x & 63;
    if (RC) {
      const int r = xb + (lane & 31), c = (d >> 3) + (lane >> 5);
      return *reinterpret_cast<const v4u*>(base + r * 128 + 16 * (c ^ (r & 7)));
    } else {
      const int g = lane >> 4, L = lane & 15;
      const int x = xb + 16 * (g & 1) + 4 * (L & 3);
      const int k = d + 8 * (g >> 1) + (L >> 2);
      const int j = x >> 3, h = (x >> 2) & 1;
      const char* p0 = base + k * (2 * X) + 16 * (j ^ (4 * (k & 3))) + 8 * h;
      const char* p1 = p0 + 4 * (2 * X);   // row k + 4 has the same swizzle
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p0));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p1));
      const v2u l2 = __builtin_bit_cast(v2u, lo), h2 = __builtin_bit_cast(v2u, hi);
      return v4u{l2[0], l2[1], h2[0], h2[1]};
    }
  }
};

// One reduction stage of the main loop, on the LDS ring slot S (a compile-time
// index, so that every LDS access names one of three distinct arrays and the
// compiler's tracking of in-flight direct-to-LDS loads can tell that reading
// slot S does not wait on the loads still filling the two other slots).
template <typename E, bool A_RC, bool B_RC, int S>
__device__ inline void stage_step(int st, int nst, char* const (&slot)[NSTAGE], const Operand<BM, A_RC>& oa,
                                  const Operand<BN, B_RC>& ob, int wm, int wn, v16f (&acc)[NI][NJ]) {
  constexpr int NL = Operand<BM, A_RC>::NQ + Operand<BN, B_RC>::NQ;   // loads per stage per thread
  // own loads of stage st complete (those of st + 1 may still fly), LDS reads drained
  if (st + 1 < nst) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(NL));
  else __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
  if (st + 2 < nst) {
    char* nb = slot[(S + 2) % NSTAGE];
    oa.issue(nb, st + 2);
    ob.issue(nb + A_BYTES, st + 2);
  }
  const char* As = slot[S];
  const char* Bs = As + A_BYTES;
  // the next reduction step's fragments are requested before the current
  // step's matrix-core work so that LDS latency overlaps the MFMAs
  v4u af[2][NI], bf[2][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i) af[0][i] = oa.frag(As, wm + 32 * i, 0);
#pragma unroll
  for (int j = 0; j < NJ; ++j) bf[0][j] = ob.frag(Bs, wn + 32 * j, 0);
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < BK / 16) {
#pragma unroll
      for (int i = 0; i < NI; ++i) af[cur ^ 1][i] = oa.frag(As, wm + 32 * i, 16 * (ks + 1));
#pragma unroll
      for (int j = 0; j < NJ; ++j) bf[cur ^ 1][j] = ob.frag(Bs, wn + 32 * j, 16 * (ks + 1));
    }
    // keep the scheduler from sinking those reads below the MFMAs (it would
    // otherwise trade the prefetch for fewer live registers)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = mfma_step<E>(af[cur][i], bf[cur][j], acc[i][j]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <typename E, bool A_RC, bool B_RC>
__global__ void __launch_bounds__(THREADS, 1) fast16dl_kernel(GemmArgs args) {
  using T = typename E::T;
  __shared__ __attribute__((aligned(1024))) char ring0[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char ring1[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char ring2[STAGE_BYTES];
  char* const slot[NSTAGE] = {ring0, ring1, ring2};

  const int64_t tiles_n = (args.cols + BN - 1) / BN;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) / tiles_n) * BM;
  const int64_t col0 = (static_cast<int64_t>(blockIdx.x) % tiles_n) * BN;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wm = (wave >> 1) * WM;
  const int wn = (wave & 1) * WN;

  Operand<BM, A_RC> oa;
  Operand<BN, B_RC> ob;
  oa.init(args.A, args.lda, row0, args.a_bytes);
  ob.init(args.B, args.ldb, col0, args.b_bytes);

  v16f acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int nst = static_cast<int>(args.red / BK);
  oa.issue(ring0, 0);
  ob.issue(ring0 + A_BYTES, 0);
  if (nst > 1) {
    oa.issue(ring1, 1);
    ob.issue(ring1 + A_BYTES, 1);
  }
  for (int st = 0; st < nst; st += NSTAGE) {
    stage_step<E, A_RC, B_RC, 0>(st, nst, slot, oa, ob, wm, wn, acc);
    if (st + 1 < nst) stage_step<E, A_RC, B_RC, 1>(st + 1, nst, slot, oa, ob, wm, wn, acc);
    if (st + 2 < nst) stage_step<E, A_RC, B_RC, 2>(st + 2, nst, slot, oa, ob, wm, wn, acc);
  }

  T* __restrict__ Y = static_cast<T*>(args.out);
  const T* __restrict__ bias = static_cast<const T*>(args.bias);
  const bool interior = row0 + BM <= args.rows && col0 + BN <= args.cols;
  const int lx = lane & 31;
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

template <typename E, bool AC, bool BC>
hipError_t launch_typed(const GemmArgs& a, hipStream_t stream) {
  const int64_t blocks = ((a.cols + BN - 1) / BN) * ((a.rows + BM - 1) / BM);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fast16dl_kernel<E, AC, BC>), dim3(static_cast<unsigned>(blocks)), dim3(THREADS), 0, stream, a);
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

}  // namespace dl

bool fast16_dl_ok(const GemmArgs& a) {
  return a.red % dl::BK == 0 && a.vec_a && a.vec_b && a.off32_a && a.off32_b;
}

hipError_t launch_fast16_dl(Op op, Dt dt, const GemmArgs& a, hipStream_t stream) {
  if (dt == DT_BF16) return dl::launch_op<BF16>(op, a, stream);
  if (dt == DT_F16) return dl::launch_op<F16>(op, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace detgemm
