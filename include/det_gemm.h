/*
 * det_gemm.h — deterministic, batch-invariant dense GEMM for training linear
 * layers on AMD Instinct MI355X (gfx950).
 *
 * The three operations of a linear layer whose weight is stored [in, out]
 * (sgemm-bi 0.1.2 PyPI page, "Use": forward, dW and dX; weight kept [in, out],
 * raw device pointers and an explicit stream at the engine boundary):
 *
 *     fwd : Y[m,n]  = X[m,k] · W[k,n] (+ bias[n])      reduction over k
 *     dx  : dX[m,k] = dY[m,n] · W[k,n]^T                reduction over n
 *     dw  : dW[k,n] = X[m,k]^T · dY[m,n]                reduction over m
 *
 * Shapes are always given as (m, k, n) of the forward problem. Every tensor is
 * dense, row-major, contiguous, and of the one dtype `dt` (bias included). All
 * pointers are device pointers on the current HIP device.
 *
 * Tiers
 *   DET_TIER_EXACT — Carbon README (alia-carbon 0.2.0), "How It Works": the
 *     reduction is cut into tiles of 32 indices anchored at 0; operands are
 *     upcast to float64; each tile's partial is an fma chain in ascending index
 *     order from +0; the tile partials are combined in ascending tile order with
 *     Neumaier's (Kahan-Babushka-Neumaier) compensation; the forward bias is
 *     added to the compensated sum in float64; the result is rounded once
 *     (round-to-nearest-even) to `dt`. The bits depend on the reduction length
 *     alone: never on m (for fwd and dx), the launch, the stream or the device
 *     state. They equal the CPU oracle's bit for bit.
 *   DET_TIER_FAST — sgemm-bi page, "Determinism contracts", tensor-core tier:
 *     matrix-core products with f32 accumulation over a fixed ascending walk of
 *     the reduction, no split of the reduction for fwd and dx, one rounding to
 *     `dt` after the bias add. Identical bits on every run; for fwd and dx the
 *     bits of a row do not depend on m. Every tile family and operand layout
 *     gives identical bits, so the library picks them for speed from the
 *     shape, m included (smaller tiles for few rows; a long-reduction
 *     forward with m >= 4096 first copies the weight transposed, 2 * k * n
 *     bytes of the stream's workspace); the bits never depend on that
 *     choice. dW of bf16/f16
 *     inputs (its reduction is over m, so batch invariance does not apply):
 *     when k x n gives few output tiles, the m rows are split into S chunks
 *     of whole 64-row stages, each accumulated from 0 in f32, and the chunk
 *     results are added in ascending chunk order before the rounding. S and
 *     the chunk length follow from (m, k, n) alone -- never from the device,
 *     the family or alignment -- so the bits stay fixed by the shape. For
 *     f32 inputs S = 1.
 *   DET_TIER_CR — Carbon README, "Roadmap", v0.2 (exact summation with a
 *     superaccumulator, independent of any order): every output is the exact
 *     real value of its dot product (plus the bias) rounded once to the output
 *     type, ties to even; an exact zero is +0; terms with an infinity or a NaN
 *     give the float64 sum of those terms. The bits are those of the exact
 *     value, so they depend on no order, tiling, m or device. Reductions of at
 *     most 2^27 - 1 (2^27 with the bias); longer ones return DET_EINVAL. The
 *     tier keeps per-row and per-column statistics and per-tile flags in the
 *     stream's workspace (4 bytes per row of each operand and per 64 x 64
 *     output tile, times 3).
 *
 * Ownership and execution
 *   The caller owns every buffer. The library keeps no reference to any of
 *   them. Some calls need device memory beyond their inputs and outputs (a
 *   workspace); the library keeps one per (device, stream):
 *     - fast tier, bf16/f16 forward with m >= 4096 and k >= 3072 or
 *       n >= 1536: a transposed
 *       copy of the weight, 2 * k * n bytes (when it cannot be had, the call
 *       runs without the copy: same bits);
 *     - fast tier, bf16/f16 dW: possibly a transposed copy of its smaller
 *       operand (2 * m * min(k, n) bytes) and, when the reduction is split
 *       (above), S * k * n * 4 bytes of f32 partials;
 *     - exact tier with at most 32 output rows (fwd and dx with m <= 32, dw
 *       with k <= 32) when 8 * rows * cols * ceil(red / 32) bytes (rows x cols
 *       the output, red the reduction length) is at most 64 MiB: every tile
 *       partial, computed in parallel (otherwise, or when the memory cannot be
 *       had, the blocked kernels run: same bits);
 *     - det_gemm_db: the float64 tile partials of up to max(2^23, 128 * n)
 *       values (m / 32 * n of them when that is less) plus 2 * n, and
 *       det_layernorm_bwd twice that for its two parameter gradients;
 *     - the correctly rounded tier: its statistics and slices (see "Tiers").
 *   The workspace is allocated (hipMalloc) on a stream's first need and
 *   replaced by a larger one when a call needs more; a replaced workspace is
 *   kept, not freed (work already enqueued may still use it), until the
 *   process ends. Those two moments allocate device memory, so they must not
 *   happen under stream capture; no call synchronises the stream or the
 *   device. Calls on one stream share its workspace in stream order; a call
 *   holds a lock of its stream from its first workspace use to its last
 *   launch, so calls from several threads on one stream do not interleave
 *   their kernels. Work is enqueued on `stream` (0 = the null stream) and
 *   the call returns once it is enqueued; the caller keeps the buffers alive
 *   until the stream has finished. Outputs must not alias inputs. Faults
 *   during execution surface at the caller's next synchronisation. The
 *   library is re-entrant; it never aborts, never prints and never changes
 *   the current device.
 *
 * Errors
 *   Every entry point returns DET_OK or a negative det_status_t; on error
 *   nothing is enqueued, and det_gemm_last_error() gives a message for the
 *   calling thread.
 */
#ifndef DET_GEMM_H
#define DET_GEMM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The *_RANGE_MIN_ and *_RANGE_MAX_ members name no dtype or tier: they make
 * every int a value of the type, so that an unknown value from a caller is a
 * defined value that the library refuses (DET_EDTYPE, DET_ETIER). */
typedef enum {
  DET_F32 = 0,   /* IEEE binary32 */
  DET_BF16 = 1,  /* bfloat16 */
  DET_F16 = 2,   /* IEEE binary16 */
  DET_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  DET_DTYPE_RANGE_MAX_ = 2147483647
} det_dtype_t;

typedef enum {
  DET_TIER_EXACT = 0, /* float64 tiles + Neumaier compensation, oracle bits */
  DET_TIER_FAST = 1,  /* matrix cores, f32 accumulate, within tolerance */
  DET_TIER_CR = 2,    /* the exact value rounded once: correctly rounded, order-free */
  DET_TIER_RANGE_MIN_ = -2147483647 - 1,
  DET_TIER_RANGE_MAX_ = 2147483647
} det_tier_t;

typedef enum {
  DET_OK = 0,
  DET_EINVAL = -1,   /* null required pointer, m/k/n < 1, or a size overflow */
  DET_EDTYPE = -2,   /* unknown dtype */
  DET_ETIER = -3,    /* unknown tier */
  DET_EDEVICE = -4,  /* current device is not gfx950, or no device */
  DET_ELAUNCH = -5   /* the runtime rejected a kernel launch or the workspace allocation */
} det_status_t;

/*
 * Forward: y[m,n] = x[m,k] · w[k,n] (+ bias[n]).
 * bias may be NULL (no bias). The exact tier adds bias to the float64
 * compensated sum before the single rounding; the fast tier adds it to the f32
 * accumulator before the rounding.
 */
det_status_t det_gemm_fwd(void* y, const void* x, const void* w, const void* bias,
                          int64_t m, int64_t k, int64_t n,
                          det_dtype_t dt, det_tier_t tier, hipStream_t stream);

/*
 * Input gradient: dx[m,k] = dy[m,n] · w[k,n]^T (reduction over n, in tiles of
 * 32 for the exact tier). Rows of dx never depend on m.
 */
det_status_t det_gemm_dx(void* dx, const void* dy, const void* w,
                         int64_t m, int64_t k, int64_t n,
                         det_dtype_t dt, det_tier_t tier, hipStream_t stream);

/*
 * Weight gradient: dw[k,n] = x[m,k]^T · dy[m,n] (reduction over the m rows,
 * in tiles of 32 rows for the exact tier; the order is fixed by m alone). The
 * fast tier with bf16/f16 inputs may split the m rows into chunks fixed by the
 * shape (see "Tiers"); a failed workspace allocation returns DET_ELAUNCH and
 * enqueues nothing. With k = 1 and x a column of ones this is the bias
 * gradient db[n].
 */
det_status_t det_gemm_dw(void* dw, const void* x, const void* dy,
                         int64_t m, int64_t k, int64_t n,
                         det_dtype_t dt, det_tier_t tier, hipStream_t stream);

/*
 * Weight gradient with an explicit output dtype: as det_gemm_dw, with dw of
 * dtype dw_dt, which must be dt or DET_F32 (f32 gradients for bf16/f16
 * training against f32 master weights: Carbon README, alia-carbon 0.2.0,
 * "Roadmap", v0.3 mixed precision). The tier's wide value is
 * rounded once to dw_dt: the exact tier's float64 compensated sum to f32, the
 * fast tier's f32 accumulation (after the ordered chunk combine when the
 * reduction is split) stored as is. dw is k x n, row-major, in dw_dt.
 * DET_EDTYPE for any other dw_dt.
 */
det_status_t det_gemm_dw_out(void* dw, det_dtype_t dw_dt, const void* x, const void* dy,
                             int64_t m, int64_t k, int64_t n,
                             det_dtype_t dt, det_tier_t tier, hipStream_t stream);

/* Size of the fixed scratch array behind det_gemm_dw_noalloc (bytes). */
#define DET_GEMM_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * det_gemm_dw_out for callers that cannot allocate device memory (code under
 * stream capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and bits as det_gemm_dw_out with the same arguments, but
 * every workspace the call needs (see "Ownership and execution") is taken from
 * one array of DET_GEMM_NOALLOC_SCRATCH_BYTES that the library holds on each
 * device (a static device allocation, kept until the process ends), and the
 * call allocates nothing. A call whose workspace would be larger returns
 * DET_EINVAL, enqueues nothing, and det_gemm_last_error() states both sizes
 * (the GPT-2-sized dW of 8192 tokens into 768 x 3072, 3072 x 768 or 768 x 2304
 * outputs fits in both tiers; a split fast-tier dW needs S * k * n * 4 bytes
 * plus 2 * m * min(k, n)). The array keeps whatever the last call left in it;
 * every kernel that reads it writes it first in the same call. All calls on one
 * device share the array, so calls that may run at the same time on one device
 * (on different streams, or from different threads without ordering) race on
 * it: order them. The call takes no stream lock. Errors as for det_gemm_dw_out;
 * DET_ELAUNCH also when the array's device address cannot be looked up.
 */
det_status_t det_gemm_dw_noalloc(void* dw, det_dtype_t dw_dt, const void* x, const void* dy,
                                 int64_t m, int64_t k, int64_t n,
                                 det_dtype_t dt, det_tier_t tier, hipStream_t stream);

/*
 * Bias gradient: db[n] = sum over i < m of dy[i, n] (sgemm-bi 0.1.2 PyPI page,
 * note after "Determinism contracts": a column sum of dY, which that engine
 * leaves to the framework). Defined here as the exact tier's
 * det_gemm_dw of a column of ones -- rows in tiles of 32, an ascending
 * float64 chain per tile, Neumaier across tiles, one rounding to db_dt (dt or
 * DET_F32) -- and computed with that arithmetic in both tiers: the operation
 * is bound by memory, so the exact sum costs nothing extra. The tile partials
 * go through the stream's workspace (see "Ownership and execution"). dy is
 * m x n, row-major, dtype dt; db has n elements of db_dt. Same errors as the
 * other entry points (DET_EDTYPE for a db_dt other than dt and DET_F32).
 */
det_status_t det_gemm_db(void* db, det_dtype_t db_dt, const void* dy, int64_t m, int64_t n,
                         det_dtype_t dt, det_tier_t tier, hipStream_t stream);

/* Largest row length det_layernorm_fwd/_bwd accept. */
#define DET_LAYERNORM_MAX_H 65536

/*
 * LayerNorm over the last dimension with float64 statistics (Carbon README,
 * alia-carbon 0.2.0, "How It Works", the LayerNorm row: mean and variance in
 * float64 instead of a thread-dependent parallel reduction). For each of the
 * `rows` rows of x (h elements, row-major, dtype dt):
 *   mean = S(x) / h,  d_j = x_j - mean,  var = S(d_j * d_j) / h   (biased),
 *   rstd = 1 / sqrt(var + eps),
 *   y_j  = round_dt((d_j * rstd) * gamma_j + beta_j),
 * where S is the exact tier's fixed-order sum (32-element tiles, an ascending
 * float64 chain in each, Neumaier across tiles) and every step is one IEEE
 * float64 operation (no fusion); a null gamma or beta skips its step. One
 * rounding to dt; the bits are fixed by the inputs alone (any row count,
 * launch or device). gamma, beta: h elements of dt, nullable. y: rows x h of
 * dt. mean, rstd: nullable float64 arrays of `rows` values (the backward
 * takes them). 1 <= h <= DET_LAYERNORM_MAX_H; eps finite and >= 0. There is
 * one arithmetic, so no tier argument. Errors as for the GEMM entry points.
 */
det_status_t det_layernorm_fwd(void* y, double* mean, double* rstd, const void* x, const void* gamma,
                               const void* beta, int64_t rows, int64_t h, double eps, det_dtype_t dt,
                               hipStream_t stream);

/*
 * Gradients of det_layernorm_fwd for the incoming gradient dy (rows x h, dt),
 * with mean and rstd as the forward returned them and xhat_j = (x_j - mean) *
 * rstd, g_j = dy_j * gamma_j (g = dy when gamma is null):
 *   dx_j     = round_dt(rstd * ((g_j - S(g) / h) - xhat_j * (S(g * xhat) / h))),
 *   dgamma_j = round_pdt(sum over rows of dy_j * xhat_j),
 *   dbeta_j  = round_pdt(sum over rows of dy_j),
 * the sums over a row (S) and over rows (in 32-row tiles, Neumaier across
 * them, as det_gemm_db) in the exact tier's fixed order. dx: rows x h of dt;
 * dgamma, dbeta: h values of param_dt (dt or DET_F32). Each output pointer is
 * nullable (that output is not computed). The parameter gradients use the
 * stream's workspace (2 * min(rows / 32, max(128, 2^23 / h)) * h float64
 * values, plus 4h between chunks). DET_EDTYPE for any other param_dt.
 */
det_status_t det_layernorm_bwd(void* dx, void* dgamma, void* dbeta, det_dtype_t param_dt, const void* dy,
                               const void* x, const double* mean, const double* rstd, const void* gamma,
                               int64_t rows, int64_t h, det_dtype_t dt, hipStream_t stream);

/* Static description of a status code. */
const char* det_gemm_strerror(det_status_t status);

/* Detail of the last error raised on the calling thread ("" if none). */
const char* det_gemm_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int det_gemm_version(void);

/*
 * Test hook: force the fast tier's tile family for later calls from any thread
 * (-1 automatic, 0 = the large family, 1 = the small family, 10 + s = tile
 * shape s of the large family's kernel where it applies: 10 = 256 x 192,
 * 11 = 128 x 192, 12 = 128 x 192 in two four-wave workgroups per compute
 * unit, 13 = 64 x 192 likewise, 14 = 128 x 192 in stages of 128, 15 =
 * 256 x 192 in four waves of 128 x 96, one per SIMD; 16 = the forward for
 * at most 32 rows of 16-bit inputs, one 32-column block per workgroup,
 * where it applies, else as 0). All
 * families produce identical bits, so this changes speed only. Returns
 * DET_EINVAL for other values.
 */
det_status_t det_gemm_debug_force_family(int family);

/*
 * Test hook: force the exact tier's kernel for later calls from any thread
 * (-1 automatic, 0 = 16x16x4 float64 matrix-core kernel with 64-row blocks of
 * 64 x 16 per wave, 1 = 16x16x4 kernel with 32 x 32 per wave and a
 * double-buffered LDS stage, 2 = float64 vector-ALU kernel, 3 = 4x4x4 float64
 * matrix-core kernel with a double-buffered LDS stage, 4 = kernel 0 with
 * 48-row blocks, 5 = the few-rows path: tile partials of every output in
 * parallel, then the ordered combine, through the stream's workspace, 6 = the
 * 4x4x4 kernel with 64-row blocks and one LDS stage, 7 = that kernel with
 * 48-row blocks). All produce the same bits (the oracle's), so this changes
 * speed only. Returns DET_EINVAL for other values.
 */
det_status_t det_gemm_debug_force_exact_kernel(int variant);

/*
 * Test hook: force the number of 32-row tiles per chunk of det_gemm_db for
 * later calls from any thread (0 = automatic: as many as fit 64 MiB of
 * float64 partials, at least 128). The chunks only bound the workspace; the
 * sum and its bits do not depend on them. Returns DET_EINVAL for tiles < 0.
 */
det_status_t det_gemm_debug_force_db_chunk(int64_t tiles);

/*
 * Test hook: the correctly rounded tier's path for every later call. 0: the
 * shape-and-data choice (16-bit inputs: 8-bit slices on the bf16 matrix
 * instructions where a tile's rows and columns span at most 40 bits, else the
 * next path); 2: 23-bit slices on the float64 matrix instructions where they
 * span at most 46 bits, else the superaccumulator; 1: the per-output
 * superaccumulator for every tile. Every path computes the exact value, so
 * this changes speed only. DET_EINVAL for other values.
 */
det_status_t det_gemm_debug_force_cr_fallback(int on);

/*
 * Test hook: the device check of every later call, from any thread, compares
 * `arch` instead of the current device's gcnArchName (NULL or "" restores the
 * device's own name). With any name other than gfx950 every entry point that
 * checks the device returns DET_EDEVICE, with det_gemm_last_error() naming
 * `arch`, and enqueues nothing -- so that the refusal a non-gfx950 device
 * gets (sgemm-bi 0.1.2 PyPI page, introduction: unsupported platforms are
 * refused with a clear message) can be exercised where the device is
 * supported. The name is copied; DET_EINVAL if it is 64 characters or longer.
 */
det_status_t det_gemm_debug_force_arch(const char* arch);

/*
 * Test hooks: the output roundings of the tiers, on the device, with the same
 * functions their epilogues call (sgemm-bi 0.1.2 PyPI page, "Determinism
 * contracts": the round-to-nearest-even downcast), so that the last step of
 * every output can be compared with a reference over chosen inputs.
 *
 * det_gemm_debug_round_f32: out[i] = the fast tier's rounding of the f32 value
 * whose bits are first + i (mod 2^32), i = 0 .. count - 1, to dt (f32: the
 * value itself). out holds count elements of dt (device memory, caller-owned).
 * DET_EINVAL if count < 0 or count > 2^32 or out is NULL with count > 0.
 *
 * det_gemm_debug_round_f64: out[i] = the exact tier's rounding of in[i]
 * (float64, device memory) to dt: round to odd at f32, then round to nearest
 * even, which equals one rounding of in[i] to dt. DET_EINVAL if count < 0 or
 * a pointer is NULL with count > 0.
 *
 * det_gemm_debug_round_f64_grouped: the same values through the LayerNorm
 * forward's rounding of eight values per lane (for bf16: round to nearest
 * even at f32 unless a lane of the wave meets an f32 result halfway between
 * two bf16 values, then round to odd at f32 for the whole group); the result
 * must equal det_gemm_debug_round_f64's. Same arguments and errors.
 *
 * All three: asynchronous on `stream`; DET_EDTYPE for an unknown dt; the device
 * check and DET_ELAUNCH as for the GEMMs.
 */
det_status_t det_gemm_debug_round_f32(void* out, uint32_t first, int64_t count, det_dtype_t dt,
                                      hipStream_t stream);
det_status_t det_gemm_debug_round_f64(void* out, const double* in, int64_t count, det_dtype_t dt,
                                      hipStream_t stream);
det_status_t det_gemm_debug_round_f64_grouped(void* out, const double* in, int64_t count, det_dtype_t dt,
                                              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DET_GEMM_H */
