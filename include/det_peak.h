/*
 * det_peak.h — peak-rate microkernels for measurement (libdetpeak.so).
 *
 * Not part of the GEMM library and not an operation of the method: a separate
 * library that the benchmark loads so that each tier's rate can be stated
 * against what the device sustains at its running clock as well as against
 * the datasheet peak. Each kernel issues the instruction a tier is built on
 * back to back, with no memory traffic.
 */
#ifndef DET_PEAK_H
#define DET_PEAK_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Runs one microkernel launch on `stream` (the current HIP device):
 *   kind 0: V_MFMA_F64_4X4X4_4B_F64 (the exact tier's float64 chains);
 *   kind 1: float64 vector fma (the exact tier's other float64 work);
 *   kind 2: V_MFMA_F32_32X32X16_BF16 (the fast tier).
 * Two workgroups of 256 threads per compute unit, `iters` (>= 1) iterations
 * each. out: device buffer of out_len doubles, at least compute units x 512;
 * every thread writes one meaningless value there (so that the arithmetic is
 * not optimised away). *flops (host memory) receives the flops the launch
 * performs; time it with events on `stream`. Returns 0, or -1 for a bad kind,
 * iters < 1, a null pointer or a short buffer, -4 when the current device is
 * not gfx950 or there is none, -5 when the launch fails. Allocates nothing.
 */
int det_peak_run(int kind, int iters, double* out, int64_t out_len, double* flops, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DET_PEAK_H */
