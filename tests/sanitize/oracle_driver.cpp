// Runs every entry point of the CPU oracle (oracle/oracle.cpp) under
// AddressSanitizer and UndefinedBehaviorSanitizer: the three GEMM ops in each
// dtype on random bit patterns (NaN, infinity, subnormals and signed zeros
// included), row subsets and the optional outputs, the correctly rounded
// GEMM, the rounding and exact-sum helpers on edge values, the LayerNorm
// forward and backward, and the refusals of invalid arguments. Buffers are
// sized exactly, so any access past them is reported. Exits non-zero on an
// unexpected return value.

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <vector>

extern "C" {
int oracle_env_ok(void);
int oracle_round(const double* r, int64_t cnt, int dt, void* out);
int oracle_gemm(int op, int dt, const void* A, const void* B, const void* bias, int64_t m, int64_t k, int64_t n,
                const int64_t* rows, int64_t nrows, void* y, double* r, double* S);
int oracle_gemm_cr(int op, int dt, const void* A, const void* B, const void* bias, int64_t m, int64_t k, int64_t n,
                   const int64_t* rows, int64_t nrows, void* y);
int oracle_exact_sum(const double* v, int64_t cnt, int dt, void* out);
int oracle_layernorm_fwd(int dt, const void* x, const void* gamma, const void* beta, int64_t rows, int64_t h,
                         double eps, void* y, double* mean, double* rstd, double* r);
int oracle_layernorm_bwd(int dt, int pdt, const void* dy, const void* x, const double* mean, const double* rstd,
                         const void* gamma, int64_t rows, int64_t h, void* dx, void* dgamma, void* dbeta,
                         double* rdx);
}

namespace {

int g_failures = 0;

void expect(int got, int want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: returned %d, expected %d\n", what, got, want);
    ++g_failures;
  }
}

uint64_t g_state = 0x9e3779b97f4a7c15ull;
uint64_t next() {   // xorshift64*
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return g_state * 0x2545f4914f6cdd1dull;
}

// n elements of dtype dt: mostly moderate values, some special bit patterns
std::vector<unsigned char> elems(int64_t n, int dt) {
  const int es = dt == 0 ? 4 : 2;
  std::vector<unsigned char> v(static_cast<size_t>(n * es));
  for (int64_t i = 0; i < n; ++i) {
    const uint64_t r = next();
    if (dt == 0) {
      uint32_t b = (r % 16 == 0) ? static_cast<uint32_t>(r >> 32) : (0x3c000000u + static_cast<uint32_t>((r >> 20) % 0x4000000u)) ^ (static_cast<uint32_t>(r) & 0x80000000u);
      std::memcpy(&v[i * 4], &b, 4);
    } else {
      uint16_t b = (r % 16 == 0) ? static_cast<uint16_t>(r >> 48)
                                 : static_cast<uint16_t>((dt == 1 ? 0x3c00u : 0x3000u) + (r >> 30) % 0x800u) ^ (static_cast<uint16_t>(r) & 0x8000u);
      std::memcpy(&v[i * 2], &b, 2);
    }
  }
  return v;
}

void gemms(int64_t m, int64_t k, int64_t n) {
  for (int dt = 0; dt < 3; ++dt) {
    const int es = dt == 0 ? 4 : 2;
    auto x = elems(m * k, dt), w = elems(k * n, dt), dy = elems(m * n, dt), bias = elems(n, dt);
    for (int op = 0; op < 3; ++op) {
      const int64_t out_rows = op == 2 ? k : m, cols = op == 1 ? k : n;
      const void* A = op == 1 ? dy.data() : x.data();
      const void* B = op == 2 ? dy.data() : w.data();
      std::vector<unsigned char> y(static_cast<size_t>(out_rows * cols * es));
      std::vector<double> r(static_cast<size_t>(out_rows * cols)), S(r.size());
      expect(oracle_gemm(op, dt, A, B, op == 0 ? bias.data() : nullptr, m, k, n, nullptr, 0, y.data(), r.data(),
                         S.data()), 0, "oracle_gemm all rows");
      const int64_t rows[2] = {out_rows - 1, 0};
      std::vector<unsigned char> y2(static_cast<size_t>(2 * cols * es));
      expect(oracle_gemm(op, dt, A, B, nullptr, m, k, n, rows, 2, y2.data(), nullptr, nullptr), 0,
             "oracle_gemm two rows");
      expect(oracle_gemm_cr(op, dt, A, B, op == 0 ? bias.data() : nullptr, m, k, n, rows, 2, y2.data()), 0,
             "oracle_gemm_cr");
      const int64_t bad_row[1] = {out_rows};
      expect(oracle_gemm(op, dt, A, B, nullptr, m, k, n, bad_row, 1, y2.data(), nullptr, nullptr), -1,
             "oracle_gemm row out of range");
    }
    expect(oracle_gemm(1, dt, x.data(), w.data(), bias.data(), m, k, n, nullptr, 0, x.data(), nullptr, nullptr), -1,
           "oracle_gemm bias on dx");
  }
}

void rounding() {
  const double inf = std::numeric_limits<double>::infinity();
  const double v[] = {0.0, -0.0, 1.0, -1.0, 1.0 + std::ldexp(1.0, -8), 1.0 + std::ldexp(1.0, -9), 65504.0, 65520.0,
                      std::ldexp(1.0, -149), std::ldexp(1.0, -150), std::ldexp(1.0, -24), std::ldexp(1.0, -25),
                      3.4028235677973366e38, 3.4e38 * 1.01, inf, -inf, std::nan(""), std::ldexp(1.0, -1074)};
  const int64_t cnt = sizeof(v) / sizeof(v[0]);
  for (int dt = 0; dt < 3; ++dt) {
    std::vector<unsigned char> out(static_cast<size_t>(cnt * (dt == 0 ? 4 : 2)));
    expect(oracle_round(v, cnt, dt, out.data()), 0, "oracle_round");
    unsigned char one[4];
    expect(oracle_exact_sum(v, 12, dt, one), 0, "oracle_exact_sum");
  }
  expect(oracle_round(v, 1, 3, nullptr), -1, "oracle_round bad dtype");
  expect(oracle_exact_sum(nullptr, 2, 0, nullptr), -1, "oracle_exact_sum null");
}

void layernorm(int64_t rows, int64_t h) {
  for (int dt = 0; dt < 3; ++dt) {
    const int es = dt == 0 ? 4 : 2;
    auto x = elems(rows * h, dt), g = elems(h, dt), b = elems(h, dt), dy = elems(rows * h, dt);
    std::vector<unsigned char> y(static_cast<size_t>(rows * h * es)), dx(y.size());
    std::vector<double> mean(static_cast<size_t>(rows)), rstd(mean.size()), r(static_cast<size_t>(rows * h)),
        rdx(r.size());
    expect(oracle_layernorm_fwd(dt, x.data(), g.data(), b.data(), rows, h, 1e-5, y.data(), mean.data(), rstd.data(),
                                r.data()), 0, "oracle_layernorm_fwd");
    expect(oracle_layernorm_fwd(dt, x.data(), nullptr, nullptr, rows, h, 0.0, y.data(), nullptr, nullptr, nullptr), 0,
           "oracle_layernorm_fwd no affine");
    for (int pdt : {dt, 0}) {
      std::vector<unsigned char> dg(static_cast<size_t>(h * (pdt == 0 ? 4 : 2))), dbt(dg.size());
      expect(oracle_layernorm_bwd(dt, pdt, dy.data(), x.data(), mean.data(), rstd.data(), g.data(), rows, h, dx.data(),
                                  dg.data(), dbt.data(), rdx.data()), 0, "oracle_layernorm_bwd");
    }
    expect(oracle_layernorm_bwd(dt, dt, dy.data(), x.data(), nullptr, rstd.data(), g.data(), rows, h, dx.data(),
                                nullptr, nullptr, nullptr), -1, "oracle_layernorm_bwd null mean");
  }
}

}  // namespace

int main() {
  if (!oracle_env_ok()) {
    std::fprintf(stderr, "FAIL floating-point environment\n");
    return 1;
  }
  gemms(1, 1, 1);
  gemms(3, 37, 5);
  gemms(17, 70, 33);
  rounding();
  layernorm(1, 1);
  layernorm(5, 70);
  std::printf("oracle driver: %d failures\n", g_failures);
  return g_failures == 0 ? 0 : 1;
}
