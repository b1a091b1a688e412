// A host-only stand-in for the HIP runtime calls and the kernel launchers that
// the C-ABI's host code uses, so that abi.cpp (argument checks, size
// arithmetic, device check, per-stream workspace and call locks, the fixed
// scratch scope) runs under AddressSanitizer and UndefinedBehaviorSanitizer on
// a machine without a GPU. "Device" memory is host memory. Every launcher reads
// every byte of its inputs and writes every byte of its outputs, as sized by
// the arguments the ABI hands it, and fills the workspace it requests, so that
// a size the ABI gets wrong against the caller's buffers, or a workspace
// shorter than requested, is reported by the sanitizer.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "common.hpp"

// Test controls, read by the drivers.
std::atomic<int> g_fake_device{0};        // what hipGetDevice reports (-1: no device)
std::atomic<long> g_fake_mallocs{0};      // hipMalloc calls so far
std::atomic<long> g_fake_fail_malloc{0};  // > 0: that many next hipMalloc calls fail

extern "C" {

hipError_t hipGetDevice(int* dev) {
  const int d = g_fake_device.load();
  if (d < 0) return hipErrorNoDevice;
  *dev = d;
  return hipSuccess;
}

// Device 0 is a gfx950 with 256 compute units; any other index is a gfx942.
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* prop, int dev) {
  std::memset(prop, 0, sizeof(*prop));
  std::strcpy(prop->gcnArchName, dev == 0 ? "gfx950:sramecc+:xnack-" : "gfx942:sramecc+:xnack-");
  prop->multiProcessorCount = dev == 0 ? 256 : 304;
  return hipSuccess;
}

hipError_t hipGetLastError(void) { return hipSuccess; }

const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "fake runtime error"; }

hipError_t hipMalloc(void** ptr, size_t bytes) {
  g_fake_mallocs.fetch_add(1);
  long f = g_fake_fail_malloc.load();
  while (f > 0) {
    if (g_fake_fail_malloc.compare_exchange_weak(f, f - 1)) return hipErrorOutOfMemory;
  }
  *ptr = std::malloc(bytes);
  return *ptr ? hipSuccess : hipErrorOutOfMemory;
}

}  // extern "C"

namespace {

unsigned read_all(const void* p, int64_t bytes) {
  unsigned s = 0;
  const unsigned char* c = static_cast<const unsigned char*>(p);
  for (int64_t i = 0; i < bytes; ++i) s += c[i];
  return s;
}

void write_all(void* p, int64_t bytes) { std::memset(p, 0x5a, static_cast<size_t>(bytes)); }

int64_t esz(detgemm::Dt dt) { return dt == detgemm::DT_F32 ? 4 : 2; }

// A workspace request like the real kernels' (partials of the split dW, the
// few-rows exact path, the correctly rounded tier's slices), filled completely.
hipError_t use_workspace(hipStream_t stream, size_t bytes) {
  void* ws = nullptr;
  const hipError_t e = detgemm::stream_workspace(stream, bytes, &ws);
  if (e != hipSuccess) return e;
  write_all(ws, static_cast<int64_t>(bytes));
  return hipSuccess;
}

std::atomic<unsigned> g_sink{0};   // keeps the reads from being optimised away

hipError_t gemm(detgemm::Dt dt, const detgemm::GemmArgs& a, size_t ws_bytes, hipStream_t stream) {
  if (ws_bytes) {
    const hipError_t e = use_workspace(stream, ws_bytes);
    if (e != hipSuccess) return e;
  }
  // operands from the output shape: A holds rows x red elements (null: a
  // column of ones), B red x cols, whatever the op's layout
  const int64_t a_bytes = a.A ? a.rows * a.red * esz(dt) : 0, b_bytes = a.red * a.cols * esz(dt);
  if (a.a_bytes != 0 && (a.a_bytes != a_bytes || a.b_bytes != b_bytes)) std::abort();
  unsigned s = (a.A ? read_all(a.A, a_bytes) : 0) + read_all(a.B, b_bytes);
  if (a.bias) s += read_all(a.bias, a.cols * esz(dt));
  g_sink.store(s, std::memory_order_relaxed);
  write_all(a.out, a.rows * a.cols * (a.out_f32 ? 4 : esz(dt)));
  return hipSuccess;
}

}  // namespace

namespace detgemm {

hipError_t launch_exact(Op, Dt dt, const GemmArgs& a, int, hipStream_t stream) {
  // the few-rows path: 8 bytes per output and 32-index tile
  const size_t ws = a.rows <= 32 ? static_cast<size_t>(8 * a.rows * a.cols * ((a.red + 31) / 32)) : 0;
  return gemm(dt, a, ws, stream);
}

hipError_t launch_fast(Op op, Dt dt, const GemmArgs& a, int, hipStream_t stream) {
  // the split dW's f32 partials (five chunks)
  const size_t ws = op == OP_DW && dt != DT_F32 ? static_cast<size_t>(5 * 4 * a.rows * a.cols) : 0;
  return gemm(dt, a, ws, stream);
}

hipError_t launch_cr(Op, Dt dt, const GemmArgs& a, int, hipStream_t stream) {
  // slices of both operands
  return gemm(dt, a, static_cast<size_t>(3 * (a.a_bytes + a.b_bytes)), stream);
}

hipError_t launch_db(Dt dt, bool out_f32, const void* dy, int64_t m, int64_t n, void* db, int64_t, hipStream_t stream) {
  const hipError_t e = use_workspace(stream, static_cast<size_t>(8 * n * ((m + 31) / 32) * 2));
  if (e != hipSuccess) return e;
  g_sink.store(read_all(dy, m * n * esz(dt)), std::memory_order_relaxed);
  write_all(db, n * (out_f32 ? 4 : esz(dt)));
  return hipSuccess;
}

hipError_t launch_layernorm_fwd(Dt dt, const void* x, const void* gamma, const void* beta, int64_t rows, int64_t h,
                                double, void* y, double* mean, double* rstd, hipStream_t) {
  unsigned s = read_all(x, rows * h * esz(dt));
  if (gamma) s += read_all(gamma, h * esz(dt));
  if (beta) s += read_all(beta, h * esz(dt));
  g_sink.store(s, std::memory_order_relaxed);
  write_all(y, rows * h * esz(dt));
  if (mean) write_all(mean, rows * 8);
  if (rstd) write_all(rstd, rows * 8);
  return hipSuccess;
}

hipError_t launch_layernorm_bwd(Dt dt, bool param_f32, const void* dy, const void* x, const double* mean,
                                const double* rstd, const void* gamma, int64_t rows, int64_t h, void* dx,
                                void* dgamma, void* dbeta, hipStream_t stream) {
  const hipError_t e = use_workspace(stream, static_cast<size_t>(16 * h * ((rows + 31) / 32)));
  if (e != hipSuccess) return e;
  unsigned s = read_all(dy, rows * h * esz(dt)) + read_all(x, rows * h * esz(dt));
  s += read_all(mean, rows * 8) + read_all(rstd, rows * 8);
  if (gamma) s += read_all(gamma, h * esz(dt));
  g_sink.store(s, std::memory_order_relaxed);
  if (dx) write_all(dx, rows * h * esz(dt));
  const int64_t p = param_f32 ? 4 : esz(dt);
  if (dgamma) write_all(dgamma, h * p);
  if (dbeta) write_all(dbeta, h * p);
  return hipSuccess;
}

hipError_t launch_round_f32(Dt dt, void* out, uint32_t, int64_t count, hipStream_t) {
  if (count > 0) write_all(out, count * esz(dt));
  return hipSuccess;
}

hipError_t launch_round_f64(Dt dt, void* out, const double* in, int64_t count, hipStream_t) {
  if (count > 0) {
    g_sink.store(read_all(in, count * 8), std::memory_order_relaxed);
    write_all(out, count * esz(dt));
  }
  return hipSuccess;
}

hipError_t launch_round_f64_grouped(Dt dt, void* out, const double* in, int64_t count, hipStream_t stream) {
  return launch_round_f64(dt, out, in, count, stream);
}

}  // namespace detgemm
