// C-ABI entry points: argument checks, device check, shape-only dispatch and
// launch on the caller's stream. The operations and their contracts are stated
// in include/det_gemm.h.

#include "../../include/det_gemm.h"

#include <atomic>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <optional>
#include <utility>
#include <vector>

#include "common.hpp"

namespace {

thread_local char g_last_error[256] = "";
std::atomic<int> g_force_family{-1};
std::atomic<int> g_force_exact{-1};
std::atomic<int64_t> g_force_db_chunk{0};
std::atomic<int> g_force_cr_fallback{0};
// longest reduction (with the bias index) of the correctly rounded tier: its
// int128 accumulator stays below 2^126 for up to 2^27 indices
constexpr int64_t kMaxCrReduction = int64_t(1) << 27;

constexpr int kMaxDevices = 64;
// 0 unknown, 1 gfx950, 2 not supported
std::atomic<int> g_device_ok[kMaxDevices];
std::atomic<int> g_device_cus[kMaxDevices];   // compute units, cached with the check

det_status_t fail(det_status_t st, const char* fmt, const char* detail = "") {
  std::snprintf(g_last_error, sizeof(g_last_error), fmt, detail);
  return st;
}

// Test hook: an architecture name that replaces the device's own in the check
// below (empty: none). Guarded by a mutex; the flag keeps the common path free
// of the lock.
std::atomic<bool> g_arch_override_on{false};
std::mutex g_arch_override_mu;
char g_arch_override[64] = "";

det_status_t check_device(int* cus) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(DET_EDEVICE, "det_gemm: no current HIP device%s");
  }
  if (dev >= kMaxDevices) return fail(DET_EDEVICE, "det_gemm: device index out of range%s");
  if (g_arch_override_on.load(std::memory_order_acquire)) {
    char arch[64];
    {
      std::lock_guard<std::mutex> lock(g_arch_override_mu);
      std::memcpy(arch, g_arch_override, sizeof(arch));
    }
    if (arch[0] != '\0' && std::strncmp(arch, "gfx950", 6) != 0)
      return fail(DET_EDEVICE, "det_gemm: device architecture %s is not gfx950 (MI355X); refusing to run", arch);
  }
  int state = g_device_ok[dev].load(std::memory_order_acquire);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(DET_EDEVICE, "det_gemm: cannot query the current device%s");
    }
    state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_device_cus[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1, std::memory_order_relaxed);
    g_device_ok[dev].store(state, std::memory_order_release);
    if (state == 2) return fail(DET_EDEVICE, "det_gemm: device architecture %s is not gfx950 (MI355X); refusing to run", prop.gcnArchName);
  }
  if (state == 2) return fail(DET_EDEVICE, "det_gemm: the current device is not gfx950 (MI355X); refusing to run%s");
  *cus = g_device_cus[dev].load(std::memory_order_relaxed);
  return DET_OK;
}

bool mul_ok(int64_t a, int64_t b, int64_t elem) {
  int64_t p;
  if (__builtin_mul_overflow(a, b, &p)) return false;
  return !__builtin_mul_overflow(p, elem, &p);
}

det_status_t run(detgemm::Op op, void* out, const void* A, const void* B, const void* bias,
                 int64_t m, int64_t k, int64_t n, det_dtype_t dt, det_tier_t tier, hipStream_t stream,
                 bool out_f32 = false) {
  g_last_error[0] = '\0';
  if (dt != DET_F32 && dt != DET_BF16 && dt != DET_F16) return fail(DET_EDTYPE, "det_gemm: unknown dtype%s");
  if (tier != DET_TIER_EXACT && tier != DET_TIER_FAST && tier != DET_TIER_CR)
    return fail(DET_ETIER, "det_gemm: unknown tier%s");
  if (!out || !A || !B) return fail(DET_EINVAL, "det_gemm: null %s pointer", !out ? "output" : "input");
  if (m < 1 || k < 1 || n < 1) return fail(DET_EINVAL, "det_gemm: m, k and n must all be >= 1%s");
  const int64_t esz = dt == DET_F32 ? 4 : 2;
  if (!mul_ok(m, k, esz) || !mul_ok(k, n, esz) || !mul_ok(m, n, esz))
    return fail(DET_EINVAL, "det_gemm: tensor size overflows int64%s");
  if (tier == DET_TIER_CR) {
    const int64_t red = (op == detgemm::OP_FWD) ? k : (op == detgemm::OP_DX ? n : m);
    if (red + 1 > kMaxCrReduction)
      return fail(DET_EINVAL, "det_gemm: the correctly rounded tier takes reductions of at most 2^27 - 1%s");
  }
  int cus = 0;
  const det_status_t dev = check_device(&cus);
  if (dev != DET_OK) return dev;

  detgemm::GemmArgs a;
  a.A = A;
  a.B = B;
  a.bias = bias;
  a.out = out;
  a.num_cu = cus;
  a.partial = nullptr;
  a.split = 1;
  a.chunk_stages = 0;
  a.out_f32 = out_f32 && dt != DET_F32;
  switch (op) {
    case detgemm::OP_FWD: a.rows = m; a.cols = n; a.red = k; a.lda = k; a.ldb = n; break;
    case detgemm::OP_DX:  a.rows = m; a.cols = k; a.red = n; a.lda = n; a.ldb = n; break;
    case detgemm::OP_DW:  a.rows = k; a.cols = n; a.red = m; a.lda = k; a.ldb = n; break;
  }
  const uintptr_t align_a = reinterpret_cast<uintptr_t>(A) | static_cast<uintptr_t>(a.lda * esz);
  const uintptr_t align_b = reinterpret_cast<uintptr_t>(B) | static_cast<uintptr_t>(a.ldb * esz);
  a.vec_a = (align_a % 16) == 0;
  a.vec_b = (align_b % 16) == 0;
  const int64_t a_elems = (op == detgemm::OP_DX) ? m * n : m * k;
  const int64_t b_elems = (op == detgemm::OP_DW) ? m * n : k * n;
  a.off32_a = a_elems * esz < (int64_t(1) << 31);
  a.off32_b = b_elems * esz < (int64_t(1) << 31);
  a.a_bytes = a_elems * esz;
  a.b_bytes = b_elems * esz;
  const detgemm::Dt d = static_cast<detgemm::Dt>(dt);
  // the stream lock guards the stream workspace; a call on a fixed buffer
  // (the entry point that allocates nothing) takes neither
  std::optional<detgemm::StreamCallLock> call_lock;
  if (!detgemm::fixed_workspace_active()) call_lock.emplace(stream);
  hipError_t err;
  if (tier == DET_TIER_EXACT) {
    const int v = g_force_exact.load(std::memory_order_relaxed);
    err = detgemm::launch_exact(op, d, a, v, stream);
  } else if (tier == DET_TIER_CR) {
    err = detgemm::launch_cr(op, d, a, g_force_cr_fallback.load(std::memory_order_relaxed), stream);
  } else {
    err = detgemm::launch_fast(op, d, a, g_force_family.load(std::memory_order_relaxed), stream);   // -1: automatic
  }
  if (err != hipSuccess) {
    size_t wanted = 0, cap = 0;
    if (err == hipErrorOutOfMemory && detgemm::fixed_workspace_overflow(&wanted, &cap)) {
      (void)hipGetLastError();
      std::snprintf(g_last_error, sizeof(g_last_error),
                    "det_gemm: this call needs %zu bytes of scratch; the fixed scratch holds %zu", wanted, cap);
      return DET_EINVAL;
    }
    return fail(DET_ELAUNCH, "det_gemm: kernel launch failed: %s", hipGetErrorString(err));
  }
  return DET_OK;
}

}  // namespace

namespace detgemm {

// det_gemm_dw_out on a fixed device buffer instead of the stream workspace:
// the arguments and the device are checked first, then `scratch` gives the
// current device's buffer (its address and size) or an error.
det_status_t dw_out_on_scratch(hipError_t (*scratch)(void** ptr, size_t* cap), void* dw, det_dtype_t dw_dt,
                               const void* x, const void* dy, int64_t m, int64_t k, int64_t n, det_dtype_t dt,
                               det_tier_t tier, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (dw_dt != dt && dw_dt != DET_F32)
    return fail(DET_EDTYPE, "det_gemm_dw_noalloc: the output dtype must be the input dtype or DET_F32%s");
  if (dt != DET_F32 && dt != DET_BF16 && dt != DET_F16) return fail(DET_EDTYPE, "det_gemm: unknown dtype%s");
  if (tier != DET_TIER_EXACT && tier != DET_TIER_FAST && tier != DET_TIER_CR)
    return fail(DET_ETIER, "det_gemm: unknown tier%s");
  int cus = 0;
  const det_status_t dev = check_device(&cus);
  if (dev != DET_OK) return dev;
  void* ptr = nullptr;
  size_t cap = 0;
  const hipError_t e = scratch(&ptr, &cap);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(DET_ELAUNCH, "det_gemm_dw_noalloc: the scratch buffer's address is not available: %s",
                hipGetErrorString(e));
  }
  FixedWorkspaceScope scope(ptr, cap);
  return run(OP_DW, dw, x, dy, nullptr, m, k, n, dt, tier, stream, dw_dt == DET_F32);
}

namespace {

// Per (device, stream) state: the call lock and the workspace.
struct StreamSlot {
  std::mutex call;          // held by a call from its first workspace request to its last launch
  void* buf = nullptr;      // current workspace
  size_t bytes = 0;
  std::vector<void*> retired;   // outgrown buffers: still possibly in use by enqueued work, never freed
};

std::mutex g_slots_mu;
// The slots and their workspaces are kept until the process ends: the map
// itself is never destroyed, so that no call racing with static destruction
// at exit finds it gone, and its buffers stay reachable.
std::map<std::pair<int, hipStream_t>, StreamSlot*>& slots() {
  static auto* m = new std::map<std::pair<int, hipStream_t>, StreamSlot*>();
  return *m;
}

StreamSlot* slot_of(int dev, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_slots_mu);
  StreamSlot*& s = slots()[{dev, stream}];
  if (!s) s = new StreamSlot();
  return s;
}

// A fixed device buffer that replaces the stream workspace for the calls of
// one thread (the entry point that allocates nothing sets it for the duration
// of its call).
struct FixedWorkspace {
  void* ptr;
  size_t cap;
  size_t wanted;   // largest request seen, for the error message
};
thread_local FixedWorkspace* t_fixed = nullptr;

}  // namespace

// Holds the calling stream's lock for the duration of one entry point's
// enqueueing, so that the launches of concurrent calls on one stream do not
// interleave (each call's kernels meet its workspace in stream order).
StreamCallLock::StreamCallLock(hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    dev = -1;
  }
  mu_ = &slot_of(dev, stream)->call;
  mu_->lock();
}
StreamCallLock::~StreamCallLock() { mu_->unlock(); }

// Workspace of at least `bytes` for (current device, stream). Calls on one
// stream are ordered by the stream (and by StreamCallLock between threads), so
// they share it; calls on different streams get different ones. Growth takes
// a new allocation of at least twice the old size and retires the old one
// without freeing it (work already enqueued may still use it), so a call
// never synchronises. Under a FixedWorkspace the fixed buffer is returned, or
// hipErrorOutOfMemory when it is too small (nothing is allocated).
hipError_t stream_workspace(hipStream_t stream, size_t bytes, void** ptr) {
  if (t_fixed) {
    if (bytes > t_fixed->wanted) t_fixed->wanted = bytes;
    if (bytes > t_fixed->cap) return hipErrorOutOfMemory;
    *ptr = t_fixed->ptr;
    return hipSuccess;
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  StreamSlot* slot = slot_of(dev, stream);   // the caller holds slot->call
  if (slot->bytes >= bytes) {
    *ptr = slot->buf;
    return hipSuccess;
  }
  const size_t grain = size_t(1) << 24;
  size_t want = (bytes + grain - 1) / grain * grain;
  if (want < 2 * slot->bytes) want = 2 * slot->bytes;
  void* p = nullptr;
  e = hipMalloc(&p, want);
  if (e != hipSuccess && want > bytes) {   // the doubling did not fit: the request itself
    (void)hipGetLastError();
    want = (bytes + grain - 1) / grain * grain;
    e = hipMalloc(&p, want);
  }
  if (e != hipSuccess) return e;
  if (slot->buf) slot->retired.push_back(slot->buf);
  slot->buf = p;
  slot->bytes = want;
  *ptr = p;
  return hipSuccess;
}

FixedWorkspaceScope::FixedWorkspaceScope(void* ptr, size_t cap) : prev_(t_fixed) {
  static_assert(sizeof(FixedWorkspace) <= sizeof(storage_) && alignof(FixedWorkspace) <= 8, "scope storage");
  t_fixed = new (storage_) FixedWorkspace{ptr, cap, 0};
}
FixedWorkspaceScope::~FixedWorkspaceScope() { t_fixed = static_cast<FixedWorkspace*>(prev_); }

bool fixed_workspace_active() { return t_fixed != nullptr; }

bool fixed_workspace_overflow(size_t* wanted, size_t* cap) {
  if (!t_fixed || t_fixed->wanted <= t_fixed->cap) return false;
  *wanted = t_fixed->wanted;
  *cap = t_fixed->cap;
  return true;
}

}  // namespace detgemm

extern "C" {

det_status_t det_gemm_fwd(void* y, const void* x, const void* w, const void* bias,
                          int64_t m, int64_t k, int64_t n,
                          det_dtype_t dt, det_tier_t tier, hipStream_t stream) {
  return run(detgemm::OP_FWD, y, x, w, bias, m, k, n, dt, tier, stream);
}

det_status_t det_gemm_dx(void* dx, const void* dy, const void* w,
                         int64_t m, int64_t k, int64_t n,
                         det_dtype_t dt, det_tier_t tier, hipStream_t stream) {
  return run(detgemm::OP_DX, dx, dy, w, nullptr, m, k, n, dt, tier, stream);
}

det_status_t det_gemm_dw(void* dw, const void* x, const void* dy,
                         int64_t m, int64_t k, int64_t n,
                         det_dtype_t dt, det_tier_t tier, hipStream_t stream) {
  return run(detgemm::OP_DW, dw, x, dy, nullptr, m, k, n, dt, tier, stream);
}

det_status_t det_gemm_dw_out(void* dw, det_dtype_t dw_dt, const void* x, const void* dy,
                             int64_t m, int64_t k, int64_t n,
                             det_dtype_t dt, det_tier_t tier, hipStream_t stream) {
  if (dw_dt != dt && dw_dt != DET_F32) {
    g_last_error[0] = '\0';
    return fail(DET_EDTYPE, "det_gemm_dw_out: the output dtype must be the input dtype or DET_F32%s");
  }
  return run(detgemm::OP_DW, dw, x, dy, nullptr, m, k, n, dt, tier, stream, dw_dt == DET_F32);
}

det_status_t det_gemm_db(void* db, det_dtype_t db_dt, const void* dy, int64_t m, int64_t n,
                         det_dtype_t dt, det_tier_t tier, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (dt != DET_F32 && dt != DET_BF16 && dt != DET_F16) return fail(DET_EDTYPE, "det_gemm: unknown dtype%s");
  if (db_dt != dt && db_dt != DET_F32)
    return fail(DET_EDTYPE, "det_gemm_db: the output dtype must be the input dtype or DET_F32%s");
  if (tier != DET_TIER_EXACT && tier != DET_TIER_FAST && tier != DET_TIER_CR)
    return fail(DET_ETIER, "det_gemm: unknown tier%s");
  if (!db || !dy) return fail(DET_EINVAL, "det_gemm: null %s pointer", !db ? "output" : "input");
  if (m < 1 || n < 1) return fail(DET_EINVAL, "det_gemm: m and n must both be >= 1%s");
  const int64_t esz = dt == DET_F32 ? 4 : 2;
  if (!mul_ok(m, n, esz)) return fail(DET_EINVAL, "det_gemm: tensor size overflows int64%s");
  if (tier == DET_TIER_CR && m + 1 > kMaxCrReduction)
    return fail(DET_EINVAL, "det_gemm: the correctly rounded tier takes reductions of at most 2^27 - 1%s");
  int cus = 0;
  const det_status_t dev = check_device(&cus);
  if (dev != DET_OK) return dev;
  detgemm::StreamCallLock call_lock(stream);
  if (tier == DET_TIER_CR) {   // the correctly rounded column sum: dW of a column of ones
    detgemm::GemmArgs a;
    std::memset(&a, 0, sizeof(a));
    a.A = nullptr;
    a.B = dy;
    a.out = db;
    a.rows = 1;
    a.cols = n;
    a.red = m;
    a.lda = 1;
    a.ldb = n;
    a.num_cu = cus;
    a.split = 1;
    a.out_f32 = db_dt == DET_F32 && dt != DET_F32;
    const hipError_t e = detgemm::launch_cr(detgemm::OP_DW, static_cast<detgemm::Dt>(dt), a,
                                            g_force_cr_fallback.load(std::memory_order_relaxed), stream);
    if (e != hipSuccess) return fail(DET_ELAUNCH, "det_gemm: kernel launch failed: %s", hipGetErrorString(e));
    return DET_OK;
  }
  const hipError_t err = detgemm::launch_db(static_cast<detgemm::Dt>(dt), db_dt == DET_F32 && dt != DET_F32, dy, m, n,
                                            db, g_force_db_chunk.load(std::memory_order_relaxed), stream);
  if (err != hipSuccess) return fail(DET_ELAUNCH, "det_gemm: kernel launch failed: %s", hipGetErrorString(err));
  return DET_OK;
}

det_status_t det_layernorm_fwd(void* y, double* mean, double* rstd, const void* x, const void* gamma,
                               const void* beta, int64_t rows, int64_t h, double eps, det_dtype_t dt,
                               hipStream_t stream) {
  g_last_error[0] = '\0';
  if (dt != DET_F32 && dt != DET_BF16 && dt != DET_F16) return fail(DET_EDTYPE, "det_layernorm: unknown dtype%s");
  if (!y || !x) return fail(DET_EINVAL, "det_layernorm: null %s pointer", !y ? "output" : "input");
  if (rows < 1 || h < 1 || h > DET_LAYERNORM_MAX_H)
    return fail(DET_EINVAL, "det_layernorm: rows must be >= 1 and h in 1 .. 65536%s");
  if (!(eps >= 0.0) || eps > 1e300) return fail(DET_EINVAL, "det_layernorm: eps must be finite and >= 0%s");
  if (!mul_ok(rows, h, dt == DET_F32 ? 4 : 2)) return fail(DET_EINVAL, "det_layernorm: tensor size overflows int64%s");
  int cus = 0;
  const det_status_t dev = check_device(&cus);
  if (dev != DET_OK) return dev;
  const hipError_t err = detgemm::launch_layernorm_fwd(static_cast<detgemm::Dt>(dt), x, gamma, beta, rows, h, eps, y,
                                                       mean, rstd, stream);
  if (err != hipSuccess) return fail(DET_ELAUNCH, "det_layernorm: kernel launch failed: %s", hipGetErrorString(err));
  return DET_OK;
}

det_status_t det_layernorm_bwd(void* dx, void* dgamma, void* dbeta, det_dtype_t param_dt, const void* dy,
                               const void* x, const double* mean, const double* rstd, const void* gamma,
                               int64_t rows, int64_t h, det_dtype_t dt, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (dt != DET_F32 && dt != DET_BF16 && dt != DET_F16) return fail(DET_EDTYPE, "det_layernorm: unknown dtype%s");
  if (param_dt != dt && param_dt != DET_F32)
    return fail(DET_EDTYPE, "det_layernorm_bwd: the parameter-gradient dtype must be the input dtype or DET_F32%s");
  if (!dy || !x || !mean || !rstd) return fail(DET_EINVAL, "det_layernorm_bwd: null %s pointer", "input");
  if (rows < 1 || h < 1 || h > DET_LAYERNORM_MAX_H)
    return fail(DET_EINVAL, "det_layernorm: rows must be >= 1 and h in 1 .. 65536%s");
  if (!mul_ok(rows, h, dt == DET_F32 ? 4 : 2)) return fail(DET_EINVAL, "det_layernorm: tensor size overflows int64%s");
  int cus = 0;
  const det_status_t dev = check_device(&cus);
  if (dev != DET_OK) return dev;
  detgemm::StreamCallLock call_lock(stream);
  const hipError_t err = detgemm::launch_layernorm_bwd(static_cast<detgemm::Dt>(dt), param_dt == DET_F32 && dt != DET_F32,
                                                       dy, x, mean, rstd, gamma, rows, h, dx, dgamma, dbeta, stream);
  if (err != hipSuccess) return fail(DET_ELAUNCH, "det_layernorm: kernel launch failed: %s", hipGetErrorString(err));
  return DET_OK;
}

const char* det_gemm_strerror(det_status_t status) {
  switch (status) {
    case DET_OK: return "success";
    case DET_EINVAL: return "invalid argument (null pointer, size < 1 or size overflow)";
    case DET_EDTYPE: return "unknown dtype";
    case DET_ETIER: return "unknown tier";
    case DET_EDEVICE: return "unsupported or missing device (gfx950 / MI355X required)";
    case DET_ELAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

const char* det_gemm_last_error(void) { return g_last_error; }

int det_gemm_version(void) { return 200; }

det_status_t det_gemm_debug_force_family(int family) {
  if (family < -1 || (family > 1 && family < 10) || family > 16)
    return fail(DET_EINVAL, "det_gemm: family must be -1, 0, 1 or 10 .. 16%s");
  g_force_family.store(family, std::memory_order_relaxed);
  return DET_OK;
}

det_status_t det_gemm_debug_force_exact_kernel(int variant) {
  if (variant < -1 || variant > 7) return fail(DET_EINVAL, "det_gemm: exact kernel must be -1 .. 7%s");
  g_force_exact.store(variant, std::memory_order_relaxed);
  return DET_OK;
}

det_status_t det_gemm_debug_force_cr_fallback(int on) {
  if (on < 0 || on > 2) return fail(DET_EINVAL, "det_gemm: cr path switch must be 0, 1 or 2%s");
  g_force_cr_fallback.store(on, std::memory_order_relaxed);
  return DET_OK;
}

det_status_t det_gemm_debug_force_arch(const char* arch) {
  if (arch != nullptr && std::strlen(arch) >= sizeof(g_arch_override))
    return fail(DET_EINVAL, "det_gemm: architecture name longer than 63 characters%s");
  std::lock_guard<std::mutex> lock(g_arch_override_mu);
  if (arch == nullptr || arch[0] == '\0') {
    g_arch_override[0] = '\0';
    g_arch_override_on.store(false, std::memory_order_release);
  } else {
    std::snprintf(g_arch_override, sizeof(g_arch_override), "%s", arch);
    g_arch_override_on.store(true, std::memory_order_release);
  }
  return DET_OK;
}

det_status_t det_gemm_debug_round_f32(void* out, uint32_t first, int64_t count, det_dtype_t dt,
                                      hipStream_t stream) {
  g_last_error[0] = '\0';
  if (dt != DET_F32 && dt != DET_BF16 && dt != DET_F16) return fail(DET_EDTYPE, "det_gemm: unknown dtype%s");
  if (count < 0 || count > (int64_t(1) << 32)) return fail(DET_EINVAL, "det_gemm_debug_round_f32: count must be in 0 .. 2^32%s");
  if (count > 0 && !out) return fail(DET_EINVAL, "det_gemm: null %s pointer", "output");
  int cus = 0;
  const det_status_t dev = check_device(&cus);
  if (dev != DET_OK) return dev;
  const hipError_t e = detgemm::launch_round_f32(static_cast<detgemm::Dt>(dt), out, first, count, stream);
  if (e != hipSuccess) return fail(DET_ELAUNCH, "det_gemm: kernel launch failed: %s", hipGetErrorString(e));
  return DET_OK;
}

static det_status_t debug_round_f64(bool grouped, void* out, const double* in, int64_t count, det_dtype_t dt,
                                    hipStream_t stream) {
  g_last_error[0] = '\0';
  if (dt != DET_F32 && dt != DET_BF16 && dt != DET_F16) return fail(DET_EDTYPE, "det_gemm: unknown dtype%s");
  if (count < 0) return fail(DET_EINVAL, "det_gemm_debug_round_f64: count must be >= 0%s");
  if (count > 0 && (!out || !in)) return fail(DET_EINVAL, "det_gemm: null %s pointer", !out ? "output" : "input");
  int cus = 0;
  const det_status_t dev = check_device(&cus);
  if (dev != DET_OK) return dev;
  const detgemm::Dt d = static_cast<detgemm::Dt>(dt);
  const hipError_t e = grouped ? detgemm::launch_round_f64_grouped(d, out, in, count, stream)
                               : detgemm::launch_round_f64(d, out, in, count, stream);
  if (e != hipSuccess) return fail(DET_ELAUNCH, "det_gemm: kernel launch failed: %s", hipGetErrorString(e));
  return DET_OK;
}

det_status_t det_gemm_debug_round_f64(void* out, const double* in, int64_t count, det_dtype_t dt,
                                      hipStream_t stream) {
  return debug_round_f64(false, out, in, count, dt, stream);
}

det_status_t det_gemm_debug_round_f64_grouped(void* out, const double* in, int64_t count, det_dtype_t dt,
                                              hipStream_t stream) {
  return debug_round_f64(true, out, in, count, dt, stream);
}

det_status_t det_gemm_debug_force_db_chunk(int64_t tiles) {
  if (tiles < 0) return fail(DET_EINVAL, "det_gemm: db chunk must be >= 0%s");
  g_force_db_chunk.store(tiles, std::memory_order_relaxed);
  return DET_OK;
}

}  // extern "C"
