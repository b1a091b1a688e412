// Drives the C-ABI's host code against the fake runtime in fake_hip.cpp, under
// AddressSanitizer and UndefinedBehaviorSanitizer: every entry point with valid
// arguments on buffers of exactly the stated sizes (each dtype, tier and op,
// shapes from 1 x 1 x 1 up), every documented refusal, calls from four threads
// on two streams that grow the stream workspaces, the fixed-scratch path and
// its overflow message, and the device checks. Exits non-zero on the first
// unexpected status; the sanitizers abort on any memory or UB error.

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "../../include/det_gemm.h"

extern std::atomic<int> g_fake_device;
extern std::atomic<long> g_fake_mallocs;
extern std::atomic<long> g_fake_fail_malloc;

namespace detgemm {
det_status_t dw_out_on_scratch(hipError_t (*scratch)(void** ptr, size_t* cap), void* dw, det_dtype_t dw_dt,
                               const void* x, const void* dy, int64_t m, int64_t k, int64_t n, det_dtype_t dt,
                               det_tier_t tier, hipStream_t stream);
}

namespace {

std::atomic<int> g_failures{0};

void expect(det_status_t got, det_status_t want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: status %d, expected %d (%s)\n", what, got, want, det_gemm_last_error());
    ++g_failures;
  } else if (want != DET_OK && det_gemm_last_error()[0] == '\0') {
    std::fprintf(stderr, "FAIL %s: refusal without a message\n", what);
    ++g_failures;
  }
}

// A buffer of exactly `bytes` bytes (ASan reports any access past it).
struct Buf {
  explicit Buf(size_t bytes) : p(std::malloc(bytes ? bytes : 1)) { std::memset(p, 1, bytes ? bytes : 1); }
  ~Buf() { std::free(p); }
  Buf(const Buf&) = delete;
  Buf& operator=(const Buf&) = delete;
  void* p;
};

size_t esz(det_dtype_t dt) { return dt == DET_F32 ? 4 : 2; }

hipStream_t stream_a = reinterpret_cast<hipStream_t>(0x1000);
hipStream_t stream_b = reinterpret_cast<hipStream_t>(0x2000);

void gemm_calls(int64_t m, int64_t k, int64_t n, det_dtype_t dt, det_tier_t tier, hipStream_t s) {
  const size_t e = esz(dt);
  Buf x(m * k * e), w(k * n * e), bias(n * e), y(m * n * e), dy(m * n * e), dx(m * k * e), dw(k * n * e),
      dw32(k * n * 4), db(n * e), db32(n * 4);
  char what[128];
  std::snprintf(what, sizeof(what), "gemm %lldx%lldx%lld dt %d tier %d", (long long)m, (long long)k, (long long)n,
                dt, tier);
  expect(det_gemm_fwd(y.p, x.p, w.p, bias.p, m, k, n, dt, tier, s), DET_OK, what);
  expect(det_gemm_fwd(y.p, x.p, w.p, nullptr, m, k, n, dt, tier, s), DET_OK, what);
  expect(det_gemm_dx(dx.p, dy.p, w.p, m, k, n, dt, tier, s), DET_OK, what);
  expect(det_gemm_dw(dw.p, x.p, dy.p, m, k, n, dt, tier, s), DET_OK, what);
  expect(det_gemm_dw_out(dw32.p, DET_F32, x.p, dy.p, m, k, n, dt, tier, s), DET_OK, what);
  expect(det_gemm_db(db.p, dt, dy.p, m, n, dt, tier, s), DET_OK, what);
  expect(det_gemm_db(db32.p, DET_F32, dy.p, m, n, dt, tier, s), DET_OK, what);
}

void layernorm_calls(int64_t rows, int64_t h, det_dtype_t dt, hipStream_t s) {
  const size_t e = esz(dt);
  Buf x(rows * h * e), g(h * e), b(h * e), y(rows * h * e), mean(rows * 8), rstd(rows * 8), dy(rows * h * e),
      dx(rows * h * e), dg(h * 4), dbt(h * 4);
  expect(det_layernorm_fwd(y.p, static_cast<double*>(mean.p), static_cast<double*>(rstd.p), x.p, g.p, b.p, rows, h,
                           1e-5, dt, s), DET_OK, "layernorm fwd");
  expect(det_layernorm_fwd(y.p, nullptr, nullptr, x.p, nullptr, nullptr, rows, h, 0.0, dt, s), DET_OK,
         "layernorm fwd, no affine");
  expect(det_layernorm_bwd(dx.p, dg.p, dbt.p, DET_F32, dy.p, x.p, static_cast<double*>(mean.p),
                           static_cast<double*>(rstd.p), g.p, rows, h, dt, s), DET_OK, "layernorm bwd f32 params");
  expect(det_layernorm_bwd(dx.p, dg.p, dbt.p, dt, dy.p, x.p, static_cast<double*>(mean.p),
                           static_cast<double*>(rstd.p), g.p, rows, h, dt, s), DET_OK, "layernorm bwd");
}

void refusals() {
  Buf x(64), w(64), y(64);
  const int64_t big = int64_t(1) << 40;
  expect(det_gemm_fwd(nullptr, x.p, w.p, nullptr, 2, 2, 2, DET_F32, DET_TIER_EXACT, stream_a), DET_EINVAL, "null out");
  expect(det_gemm_fwd(y.p, nullptr, w.p, nullptr, 2, 2, 2, DET_F32, DET_TIER_EXACT, stream_a), DET_EINVAL, "null x");
  expect(det_gemm_dx(y.p, x.p, nullptr, 2, 2, 2, DET_F32, DET_TIER_FAST, stream_a), DET_EINVAL, "null w");
  expect(det_gemm_fwd(y.p, x.p, w.p, nullptr, 0, 2, 2, DET_F32, DET_TIER_EXACT, stream_a), DET_EINVAL, "m = 0");
  expect(det_gemm_dw(y.p, x.p, w.p, 2, -3, 2, DET_F32, DET_TIER_EXACT, stream_a), DET_EINVAL, "k < 0");
  expect(det_gemm_fwd(y.p, x.p, w.p, nullptr, big, big, 2, DET_BF16, DET_TIER_EXACT, stream_a), DET_EINVAL,
         "size overflow");
  expect(det_gemm_fwd(y.p, x.p, w.p, nullptr, 2, 2, 2, static_cast<det_dtype_t>(7), DET_TIER_EXACT, stream_a),
         DET_EDTYPE, "bad dtype");
  expect(det_gemm_fwd(y.p, x.p, w.p, nullptr, 2, 2, 2, DET_F32, static_cast<det_tier_t>(9), stream_a), DET_ETIER,
         "bad tier");
  expect(det_gemm_dw(y.p, x.p, w.p, int64_t(1) << 27, 1, 1, DET_BF16, DET_TIER_CR, stream_a), DET_EINVAL,
         "cr reduction too long");
  expect(det_gemm_dw_out(y.p, DET_F16, x.p, w.p, 2, 2, 2, DET_BF16, DET_TIER_EXACT, stream_a), DET_EDTYPE,
         "dw_out dtype");
  expect(det_gemm_db(y.p, DET_BF16, x.p, 2, 2, DET_F16, DET_TIER_EXACT, stream_a), DET_EDTYPE, "db dtype");
  expect(det_gemm_db(y.p, DET_F32, x.p, 0, 2, DET_F32, DET_TIER_EXACT, stream_a), DET_EINVAL, "db m = 0");
  expect(det_layernorm_fwd(y.p, nullptr, nullptr, x.p, nullptr, nullptr, 1, DET_LAYERNORM_MAX_H + 1, 1e-5, DET_F32,
                           stream_a), DET_EINVAL, "layernorm h too large");
  expect(det_layernorm_fwd(y.p, nullptr, nullptr, x.p, nullptr, nullptr, 1, 4, -1.0, DET_F32, stream_a), DET_EINVAL,
         "layernorm eps < 0");
  expect(det_layernorm_bwd(y.p, nullptr, nullptr, DET_F32, x.p, x.p, nullptr, nullptr, nullptr, 1, 4, DET_F32,
                           stream_a), DET_EINVAL, "layernorm bwd null statistics");
  expect(det_gemm_debug_force_family(99), DET_EINVAL, "family out of range");
  expect(det_gemm_debug_force_exact_kernel(99), DET_EINVAL, "exact kernel out of range");
  const std::string long_name(64, 'x');
  expect(det_gemm_debug_force_arch(long_name.c_str()), DET_EINVAL, "arch name of 64 characters");
}

void rounding_hooks() {
  for (int dt = 0; dt < 3; ++dt) {
    Buf out(1000 * esz(static_cast<det_dtype_t>(dt))), in(1000 * 8);
    expect(det_gemm_debug_round_f32(out.p, 0xfffffff0u, 1000, static_cast<det_dtype_t>(dt), stream_a), DET_OK,
           "round f32");
    expect(det_gemm_debug_round_f64(out.p, static_cast<const double*>(in.p), 1000, static_cast<det_dtype_t>(dt),
                                    stream_a), DET_OK, "round f64");
    expect(det_gemm_debug_round_f64_grouped(out.p, static_cast<const double*>(in.p), 1000,
                                            static_cast<det_dtype_t>(dt), stream_a), DET_OK, "round f64 grouped");
  }
  expect(det_gemm_debug_round_f32(nullptr, 0, 0, DET_BF16, stream_a), DET_OK, "round f32, nothing");
  expect(det_gemm_debug_round_f32(nullptr, 0, 5, DET_BF16, stream_a), DET_EINVAL, "round f32, null out");
  expect(det_gemm_debug_round_f32(nullptr, 0, (int64_t(1) << 32) + 1, DET_BF16, stream_a), DET_EINVAL,
         "round f32, count > 2^32");
  expect(det_gemm_debug_round_f64(nullptr, nullptr, -1, DET_F16, stream_a), DET_EINVAL, "round f64, count < 0");
  expect(det_gemm_debug_round_f64(nullptr, nullptr, 3, DET_F16, stream_a), DET_EINVAL, "round f64, null");
  expect(det_gemm_debug_round_f64_grouped(nullptr, nullptr, 3, DET_BF16, stream_a), DET_EINVAL,
         "round f64 grouped, null");
  expect(det_gemm_debug_round_f64(nullptr, nullptr, 0, static_cast<det_dtype_t>(-9), stream_a), DET_EDTYPE,
         "round f64, bad dtype");
}

void devices() {
  Buf x(64), w(64), y(64);
  expect(det_gemm_debug_force_arch("gfx942"), DET_OK, "force arch");
  expect(det_gemm_fwd(y.p, x.p, w.p, nullptr, 2, 2, 2, DET_F32, DET_TIER_EXACT, stream_a), DET_EDEVICE,
         "forced gfx942");
  expect(det_gemm_debug_force_arch(nullptr), DET_OK, "restore arch");
  g_fake_device = 1;   // a gfx942
  expect(det_gemm_fwd(y.p, x.p, w.p, nullptr, 2, 2, 2, DET_F32, DET_TIER_EXACT, stream_a), DET_EDEVICE, "gfx942");
  expect(det_gemm_fwd(y.p, x.p, w.p, nullptr, 2, 2, 2, DET_F32, DET_TIER_EXACT, stream_a), DET_EDEVICE,
         "gfx942, cached");
  g_fake_device = -1;  // none
  expect(det_gemm_fwd(y.p, x.p, w.p, nullptr, 2, 2, 2, DET_F32, DET_TIER_EXACT, stream_a), DET_EDEVICE, "no device");
  g_fake_device = 70;  // past the library's device table
  expect(det_gemm_fwd(y.p, x.p, w.p, nullptr, 2, 2, 2, DET_F32, DET_TIER_EXACT, stream_a), DET_EDEVICE,
         "device index out of range");
  g_fake_device = 0;
}

// the fixed scratch of the entry point that allocates nothing
char g_scratch[4096];
size_t g_scratch_cap = sizeof(g_scratch);
hipError_t small_scratch(void** ptr, size_t* cap) {
  *ptr = g_scratch;
  *cap = g_scratch_cap;
  return hipSuccess;
}

void fixed_scratch() {
  Buf x(16 * 8 * 2), dy(16 * 8 * 2), dw(8 * 8 * 4);
  const long before = g_fake_mallocs.load();
  // the fast tier's split dW wants 5 x 4 x 8 x 8 = 1280 bytes: fits
  expect(detgemm::dw_out_on_scratch(small_scratch, dw.p, DET_F32, x.p, dy.p, 16, 8, 8, DET_BF16, DET_TIER_FAST,
                                    stream_a), DET_OK, "fixed scratch");
  g_scratch_cap = 1000;
  expect(detgemm::dw_out_on_scratch(small_scratch, dw.p, DET_F32, x.p, dy.p, 16, 8, 8, DET_BF16, DET_TIER_FAST,
                                    stream_a), DET_EINVAL, "fixed scratch too small");
  if (!std::strstr(det_gemm_last_error(), "1280")) {
    std::fprintf(stderr, "FAIL fixed scratch message: %s\n", det_gemm_last_error());
    ++g_failures;
  }
  g_scratch_cap = sizeof(g_scratch);
  if (g_fake_mallocs.load() != before) {
    std::fprintf(stderr, "FAIL the fixed-scratch path allocated\n");
    ++g_failures;
  }
  // after the scope, the same thread's calls use the stream workspace again
  Buf dwb(8 * 8 * 2);
  expect(det_gemm_dw(dwb.p, x.p, dy.p, 16, 8, 8, DET_BF16, DET_TIER_FAST, stream_a), DET_OK, "after fixed scratch");
}

void failed_allocation() {
  // a workspace the runtime cannot give is reported, and the next call works
  Buf x(40 * 3000 * 2), dy(40 * 3000 * 2), dw(3000 * 3000 * 2);
  g_fake_fail_malloc = 2;
  expect(det_gemm_dw(dw.p, x.p, dy.p, 40, 3000, 3000, DET_BF16, DET_TIER_FAST,
                     reinterpret_cast<hipStream_t>(0x3000)), DET_ELAUNCH, "workspace allocation fails");
  g_fake_fail_malloc = 0;
  expect(det_gemm_dw(dw.p, x.p, dy.p, 40, 3000, 3000, DET_BF16, DET_TIER_FAST,
                     reinterpret_cast<hipStream_t>(0x3000)), DET_OK, "after a failed allocation");
}

void threads() {
  std::vector<std::thread> ts;
  std::atomic<int> bad{0};
  for (int t = 0; t < 4; ++t) {
    ts.emplace_back([t, &bad]() {
      const hipStream_t s = (t & 1) ? stream_a : stream_b;
      for (int i = 0; i < 60; ++i) {
        const int64_t m = 1 + (i * 7 + t) % 40, k = 1 + (i * 13) % 300, n = 1 + (i * 5 + 3 * t) % 200;
        const int before = g_failures.load();
        gemm_calls(m, k, n, static_cast<det_dtype_t>(i % 3), static_cast<det_tier_t>((i + t) % 3), s);
        if (g_failures.load() != before) bad.fetch_add(1);
      }
    });
  }
  for (auto& th : ts) th.join();
  if (bad.load()) ++g_failures;
}

}  // namespace

int main() {
  for (int dt = 0; dt < 3; ++dt)
    for (int tier = 0; tier < 3; ++tier)
      for (const auto& s : std::vector<std::vector<int64_t>>{{1, 1, 1}, {5, 7, 3}, {33, 64, 17}, {300, 129, 65}})
        gemm_calls(s[0], s[1], s[2], static_cast<det_dtype_t>(dt), static_cast<det_tier_t>(tier), stream_a);
  for (int dt = 0; dt < 3; ++dt) {
    layernorm_calls(1, 1, static_cast<det_dtype_t>(dt), stream_a);
    layernorm_calls(37, 300, static_cast<det_dtype_t>(dt), stream_b);
  }
  refusals();
  rounding_hooks();
  devices();
  fixed_scratch();
  failed_allocation();
  threads();
  if (det_gemm_version() <= 0 || !det_gemm_strerror(DET_EINVAL)) ++g_failures;
  std::printf("abi driver: %d failures\n", g_failures.load());
  return g_failures.load() == 0 ? 0 : 1;
}
