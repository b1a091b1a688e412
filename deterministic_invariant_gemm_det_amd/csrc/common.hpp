// Internal definitions shared by the library's HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

#include <mutex>

namespace detgemm {

enum Op { OP_FWD = 0, OP_DX = 1, OP_DW = 2 };

// One GEMM launch, already mapped onto "output rows x output cols, reduction red":
//   out[r][c] = sum_l A(r, l) * B(l, c)  (+ bias[c])
// with A(r, l) = A[r * lda + l] when a_red_contig, else A[l * lda + r];
//      B(l, c) = B[c * ldb + l] when b_red_contig, else B[l * ldb + c].
struct GemmArgs {
  const void* A;
  const void* B;
  const void* bias;  // nullable, [cols]
  void* out;         // [rows][cols], leading dimension cols
  int64_t lda, ldb;
  int64_t rows, cols, red;
  bool vec_a, vec_b; // 16-byte vector loads allowed (base and row stride aligned)
  bool off32_a, off32_b; // every element offset of the operand fits in 32 bits
  int64_t a_bytes, b_bytes; // size of each operand in bytes
  int num_cu;        // compute units of the device (launch-shape choice only)
  // Fast tier, dW of 16-bit inputs: the reduction is split into `split` chunks
  // of `chunk_stages` stages of 64; chunk c writes its f32 partial outputs to
  // partial + c * rows * cols (row-major). partial == nullptr: no split.
  float* partial;
  int split;
  int chunk_stages;
  // dW only: write f32 outputs (rounded once from the tier's wide value)
  // instead of the input dtype
  bool out_f32;
};

enum Dt { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

// ---- element types: exact upcast and the final single rounding -------------

struct F32 {
  using T = float;
  __device__ static inline double up(T v) { return static_cast<double>(v); }
  __device__ static inline float to_f32(T v) { return v; }
};
struct BF16 {
  using T = uint16_t;  // raw bfloat16 bits
  __device__ static inline double up(T v) { return static_cast<double>(__uint_as_float(static_cast<uint32_t>(v) << 16)); }
  __device__ static inline float to_f32(T v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
};
struct F16 {
  using T = _Float16;
  __device__ static inline double up(T v) { return static_cast<double>(static_cast<float>(v)); }
  __device__ static inline float to_f32(T v) { return static_cast<float>(v); }
};

// float64 -> float32 rounded to odd: the truncation toward zero, with its last
// bit set when the conversion was inexact (Boldo and Melquiond, "Emulation of
// FMA and correctly rounded sums: proved algorithms using rounding to odd",
// IEEE TC 2008). A second rounding from the result to any format with at least
// two fewer significand bits equals a single rounding from float64.
__device__ inline float f64_to_f32_odd(double r) {
  const float f = static_cast<float>(r);  // round to nearest even
  const uint32_t u = __float_as_uint(f);
  const double back = static_cast<double>(f);
  // inexact: step to the neighbour toward zero if the rounding went away from
  // zero, then set the last bit (selects rather than branches; a NaN stays NaN)
  const bool inexact = back != r;
  const uint32_t down = (inexact && __builtin_fabs(back) > __builtin_fabs(r)) ? 1u : 0u;
  return __uint_as_float((u - down) | (inexact ? 1u : 0u));
}

// Single round-to-nearest-even of a float64 value to the output type: for
// bf16 and f16 round to odd at float32, then the hardware conversion
// (V_CVT_PK_BF16_F32 / V_CVT_F16_F32, round to nearest even, subnormals kept).
template <typename E> __device__ inline typename E::T round_from_f64(double r);
template <> __device__ inline float round_from_f64<F32>(double r) { return static_cast<float>(r); }
template <> __device__ inline uint16_t round_from_f64<BF16>(double r) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f64_to_f32_odd(r)));
}
template <> __device__ inline _Float16 round_from_f64<F16>(double r) { return static_cast<_Float16>(f64_to_f32_odd(r)); }

// N float64 values each rounded once, as round_from_f64 does, with fewer
// float64 operations for bf16: round to nearest even at float32, then the
// hardware conversion. Rounding to nearest is monotone and every midpoint
// between neighbouring bf16 values is a float32 value, so the two roundings
// equal one unless the float32 result is such a midpoint (its low 16 bits are
// 0x8000). If any lane of the wave meets that case, the whole group takes the
// round-to-odd path (one branch for the wave, rarely taken). f16 and f32 use
// round_from_f64 as it stands.
template <typename E, int N>
__device__ inline void round_group(const double (&u)[N], typename E::T (&out)[N]) {
  if constexpr (std::is_same<E, BF16>::value) {
    float f[N];
    bool tie = false;
#pragma unroll
    for (int e = 0; e < N; ++e) {
      f[e] = static_cast<float>(u[e]);
      tie |= (__float_as_uint(f[e]) & 0xffffu) == 0x8000u;
    }
    if (__builtin_amdgcn_ballot_w64(tie) != 0) {
#pragma unroll
      for (int e = 0; e < N; ++e) f[e] = f64_to_f32_odd(u[e]);
    }
#pragma unroll
    for (int e = 0; e < N; ++e) out[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(f[e]));
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) out[e] = round_from_f64<E>(u[e]);
  }
}

// Round-to-nearest-even of an f32 accumulator to the output type.
template <typename E> __device__ inline typename E::T round_from_f32(float r);
template <> __device__ inline float round_from_f32<F32>(float r) { return r; }
template <> __device__ inline uint16_t round_from_f32<BF16>(float r) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(r));   // V_CVT_PK_BF16_F32, round to nearest even
}
template <> __device__ inline _Float16 round_from_f32<F16>(float r) { return static_cast<_Float16>(r); }

// Host-side launchers (one per tier), defined next to their kernels.
hipError_t launch_exact(Op op, Dt dt, const GemmArgs& a, int variant, hipStream_t stream);
hipError_t launch_fast(Op op, Dt dt, const GemmArgs& a, int family, hipStream_t stream);
hipError_t launch_fast16(Op op, Dt dt, const GemmArgs& a, int family, hipStream_t stream);
bool fast16_w_ok(const GemmArgs& a);
int fast16_w_shape(int64_t cols, int64_t red);
hipError_t launch_fast16_w(Op op, Dt dt, const GemmArgs& a, int shape, hipStream_t stream);
int fast_auto_family(Op op, Dt dt, int64_t cols, int64_t red);
// Forward of 16-bit inputs with at most 32 rows: one 32-column block per
// workgroup streaming the weight (skinny.hip); same bits as the tiled kernels.
bool fast16_skinny_ok(const GemmArgs& a);
hipError_t launch_fast16_skinny(Dt dt, const GemmArgs& a, hipStream_t stream);

// Split of the fast tier's dW reduction (16-bit inputs), from the shape only:
// returns the chunk count S >= 1 and sets *chunk_stages.
int fast_dw_split(int64_t m, int64_t k, int64_t n, int* chunk_stages);
// out[i] = round(((P_0[i] + P_1[i]) + ...) + P_{S-1}[i]) over `count` elements, P_c = partial + c * count.
hipError_t launch_combine(Dt dt, bool out_f32, const float* partial, int split, int64_t count, void* out,
                          hipStream_t stream);
// db[n] = sum_i dy[i, n] with the exact tier's arithmetic (the dW of a column of ones).
// chunk_tiles > 0 forces the tiles per chunk of the column sum (bits unchanged)
hipError_t launch_db(Dt dt, bool out_f32, const void* dy, int64_t m, int64_t n, void* db, int64_t chunk_tiles,
                     hipStream_t stream);
// LayerNorm over rows of h elements (h <= 65536), float64 statistics.
hipError_t launch_layernorm_fwd(Dt dt, const void* x, const void* gamma, const void* beta, int64_t rows, int64_t h,
                                double eps, void* y, double* mean, double* rstd, hipStream_t stream);
hipError_t launch_layernorm_bwd(Dt dt, bool param_f32, const void* dy, const void* x, const double* mean,
                                const double* rstd, const void* gamma, int64_t rows, int64_t h, void* dx,
                                void* dgamma, void* dbeta, hipStream_t stream);
// Test hooks: round_from_f32 on the f32 values with bits first, first + 1, ...
// (count of them, wrapping at 2^32) and round_from_f64 on in[0 .. count - 1].
hipError_t launch_round_f32(Dt dt, void* out, uint32_t first, int64_t count, hipStream_t stream);
hipError_t launch_round_f64(Dt dt, void* out, const double* in, int64_t count, hipStream_t stream);
hipError_t launch_round_f64_grouped(Dt dt, void* out, const double* in, int64_t count, hipStream_t stream);
// Correctly rounded tier; a null A stands for a column of ones.
hipError_t launch_cr(Op op, Dt dt, const GemmArgs& a, int force_fallback, hipStream_t stream);
// A device workspace of at least `bytes` for (current device, stream), owned
// by the library; the caller holds that stream's StreamCallLock.
hipError_t stream_workspace(hipStream_t stream, size_t bytes, void** ptr);
// Held by every entry point while it requests workspace and enqueues its
// kernels: one lock per (device, stream).
class StreamCallLock {
 public:
  explicit StreamCallLock(hipStream_t stream);
  ~StreamCallLock();
  StreamCallLock(const StreamCallLock&) = delete;
  StreamCallLock& operator=(const StreamCallLock&) = delete;

 private:
  std::mutex* mu_;
};
// While one lives on a thread, every workspace request of that thread's calls
// gets `ptr` (cap bytes of device memory) instead of the stream workspace, or
// hipErrorOutOfMemory when it asks for more; nothing is allocated.
class FixedWorkspaceScope {
 public:
  FixedWorkspaceScope(void* ptr, size_t cap);
  ~FixedWorkspaceScope();
  FixedWorkspaceScope(const FixedWorkspaceScope&) = delete;
  FixedWorkspaceScope& operator=(const FixedWorkspaceScope&) = delete;

 private:
  void* prev_;
  alignas(8) unsigned char storage_[32];
};
bool fixed_workspace_active();
// true when a request of the current scope exceeded its buffer (the largest
// request and the buffer's size are returned)
bool fixed_workspace_overflow(size_t* wanted, size_t* cap);

}  // namespace detgemm
