// Plain CPU oracle for the deterministic, batch-invariant GEMM.
//
// TEST INFRASTRUCTURE ONLY. Nothing in the GPU library links, includes or
// calls this file; only the test suite, the smoke check and the CPU-baseline
// leg of the benchmark load the shared object built from it. It shares no
// code, header, table or helper with the GPU kernels.
//
// It is deliberately slow and single-threaded: every output element is one
// call of kbn_dot(), written straight from the definition below.
//
// What is computed
// ----------------
// Carbon README (alia-carbon 0.2.0), "How It Works": a matmul is split into
// tiles, the operands are upcast to float64, and the tile results are
// accumulated with Kahan-Babushka-Neumaier (KBN) compensation in a fixed order.
// The page leaves the tile geometry and the within-tile order open; the
// readings taken here:
//   * the reduction index is cut into tiles of KT = 32 consecutive indices,
//     anchored at index 0; the last tile may be short;
//   * inside tile t the partial is p_t = +0.0 followed by p_t = fma(a_k, b_k, p_t)
//     for k ascending (every product of two upcast f32/bf16/f16 values is exact
//     in float64, so each step rounds once);
//   * across tiles, Neumaier's variant of compensated summation, in ascending
//     tile order, from (s, c) = (+0.0, +0.0); the result is r = s + c;
//   * the forward bias is added after the compensated sum, r = r + b_j, in
//     float64;
//   * the output is a single round-to-nearest-even from float64 to the output
//     dtype (sgemm-bi 0.1.2 PyPI page, "Determinism contracts", names an RNE
//     downcast; here it is applied once, from float64).
//
// The three operations (sgemm-bi page, "Use": forward, dW and dX of a linear
// layer whose weight is stored [in, out]):
//   fwd: Y[i,j]  = sum_k X[i,k]  * W[k,j]   (+ b[j])   reduction over k < K
//   dx : dX[i,q] = sum_n dY[i,n] * W[q,n]              reduction over n < N
//   dw : dW[q,j] = sum_i X[i,q]  * dY[i,j]             reduction over i < M
//
// Alongside each output the oracle can return r (the float64 value before the
// downcast) and S = sum |a_k * b_k| + |b_j|, which bound the fast tier's error.
//
// The correctly rounded tier (Carbon README, "Roadmap", v0.2: exact summation
// with a superaccumulator, independent of order) is defined separately below:
// oracle_gemm_cr rounds the exact value of each dot product once.
//
// LayerNorm (Carbon README, "How It Works", the LayerNorm row: mean and
// variance in float64 instead of a thread-dependent parallel reduction) is
// defined on top of the same summation; see oracle_layernorm_fwd/_bwd below.

#include <cfenv>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>
#include <algorithm>
#include <xmmintrin.h>

namespace {

enum Dtype { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };
enum Op { OP_FWD = 0, OP_DX = 1, OP_DW = 2 };
constexpr int64_t KT = 32;  // tile width along the reduction index

// ---- exact decode of one stored element into float64 ------------------------

double decode_f16(uint16_t h) {
  const int sign = h >> 15;
  const int e = (h >> 10) & 0x1f;
  const int m = h & 0x3ff;
  double v;
  if (e == 0) {
    v = std::ldexp(static_cast<double>(m), -24);              // zero or subnormal
  } else if (e == 0x1f) {
    v = m ? std::nan("") : HUGE_VAL;                          // NaN or infinity
  } else {
    v = std::ldexp(static_cast<double>(1024 + m), e - 25);    // normal
  }
  return sign ? -v : v;
}

double decode_bf16(uint16_t h) {
  const uint32_t u = static_cast<uint32_t>(h) << 16;  // bf16 is the top half of an f32
  float f;
  std::memcpy(&f, &u, 4);
  return static_cast<double>(f);
}

double decode(const void* base, int64_t idx, int dt) {
  if (dt == DT_F32) {
    float f;
    std::memcpy(&f, static_cast<const char*>(base) + 4 * idx, 4);
    return static_cast<double>(f);
  }
  uint16_t h;
  std::memcpy(&h, static_cast<const char*>(base) + 2 * idx, 2);
  return dt == DT_BF16 ? decode_bf16(h) : decode_f16(h);
}

// ---- single round-to-nearest-even from float64 to the output dtype ----------
//
// For the 16-bit formats the rounding is a search in an exhaustive table of
// every finite non-negative encoding (codes 0 .. max_finite, whose values
// increase with the code). Ties go to the code with an even last bit. Values
// at or beyond max_finite + half an ulp go to infinity, as IEEE RNE does.

struct Table16 {
  std::vector<double> val;   // val[code] for code = 0 .. max_finite
  uint16_t max_finite;
  uint16_t inf_code;
  uint16_t nan_code;
  double beyond;             // the value the next code would have (2^(emax+1))
};

Table16 make_table(int dt) {
  Table16 t;
  if (dt == DT_BF16) {
    t.max_finite = 0x7f7f; t.inf_code = 0x7f80; t.nan_code = 0x7fc0; t.beyond = std::ldexp(1.0, 128);
  } else {
    t.max_finite = 0x7bff; t.inf_code = 0x7c00; t.nan_code = 0x7e00; t.beyond = std::ldexp(1.0, 16);
  }
  for (uint32_t code = 0; code <= t.max_finite; ++code) {
    const uint16_t h = static_cast<uint16_t>(code);
    t.val.push_back(dt == DT_BF16 ? decode_bf16(h) : decode_f16(h));
  }
  return t;
}

const Table16& table(int dt) {
  static const Table16 bf = make_table(DT_BF16);
  static const Table16 hf = make_table(DT_F16);
  return dt == DT_BF16 ? bf : hf;
}

uint16_t round_to_16(double r, int dt) {
  const Table16& t = table(dt);
  if (std::isnan(r)) return t.nan_code;
  const uint16_t sign = std::signbit(r) ? 0x8000 : 0;
  const double a = std::fabs(r);
  // lo = largest code whose value is <= a
  const auto it = std::upper_bound(t.val.begin(), t.val.end(), a);
  const uint16_t lo = static_cast<uint16_t>((it - t.val.begin()) - 1);
  if (t.val[lo] == a) return static_cast<uint16_t>(lo | sign);
  const bool lo_is_max = (lo == t.max_finite);
  const uint16_t hi = lo_is_max ? t.inf_code : static_cast<uint16_t>(lo + 1);
  const double v_hi = lo_is_max ? t.beyond : t.val[hi];
  // Both sums below are exact in float64 (the table holds 8- or 11-bit values).
  const double twice = 2.0 * a;
  const double mid2 = t.val[lo] + v_hi;
  uint16_t code;
  if (twice < mid2) code = lo;
  else if (twice > mid2) code = hi;
  else code = (lo % 2 == 0) ? lo : hi;
  return static_cast<uint16_t>(code | sign);
}

void store(void* out, int64_t idx, double r, int dt) {
  if (dt == DT_F32) {
    const float f = static_cast<float>(r);  // RNE under the default environment
    std::memcpy(static_cast<char*>(out) + 4 * idx, &f, 4);
  } else {
    const uint16_t h = round_to_16(r, dt);
    std::memcpy(static_cast<char*>(out) + 2 * idx, &h, 2);
  }
}

// ---- the compensated tiled dot product (the whole method for one output) ----
//
// a[0..L) and b[0..L) are the two operand sequences along the reduction index,
// already upcast to float64. Returns r = s + c; *S receives sum |a_k * b_k|.

double kbn_dot(const double* a, const double* b, int64_t L, double* S) {
  double s = +0.0;
  double c = +0.0;
  double abs_sum = 0.0;
  for (int64_t t0 = 0; t0 < L; t0 += KT) {
    const int64_t t1 = std::min(t0 + KT, L);
    double p = +0.0;                        // tile partial p_t
    for (int64_t k = t0; k < t1; ++k) {
      p = std::fma(a[k], b[k], p);
      abs_sum = abs_sum + std::fabs(a[k] * b[k]);
    }
    // Neumaier's update of (s, c) with the next tile partial
    const double tt = s + p;
    if (std::fabs(s) >= std::fabs(p)) {
      c = c + ((s - tt) + p);
    } else {
      c = c + ((p - tt) + s);
    }
    s = tt;
  }
  *S = abs_sum;
  return s + c;
}

}  // namespace

extern "C" {

int oracle_version(void) { return 3; }

// 1 when the floating-point environment is the IEEE default this oracle needs:
// round-to-nearest-even, no flush-to-zero, no denormals-are-zero.
int oracle_env_ok(void) {
  const unsigned csr = _mm_getcsr();
  const bool ftz = (csr & 0x8000u) != 0;
  const bool daz = (csr & 0x0040u) != 0;
  return (std::fegetround() == FE_TONEAREST && !ftz && !daz) ? 1 : 0;
}

// Round cnt float64 values to dtype dt (raw bits out: f32 as 4 bytes, bf16/f16 as 2).
int oracle_round(const double* r, int64_t cnt, int dt, void* out) {
  if (dt < DT_F32 || dt > DT_F16 || cnt < 0 || (cnt > 0 && (!r || !out))) return -1;
  for (int64_t i = 0; i < cnt; ++i) store(out, i, r[i], dt);
  return 0;
}

// Evaluate rows of one GEMM output.
//   op   : 0 fwd (A = X[m,k], B = W[k,n], out Y[m,n], bias[n] nullable)
//          1 dx  (A = dY[m,n], B = W[k,n], out dX[m,k])
//          2 dw  (A = X[m,k], B = dY[m,n], out dW[k,n])
//   rows : output row indices to evaluate (NULL: all output rows, in order)
//   y    : nrows x cols output, raw bits of dtype dt
//   r, S : nullable nrows x cols float64 (value before rounding; abs-sum bound)
// Returns 0, or -1 on invalid arguments.
int oracle_gemm(int op, int dt, const void* A, const void* B, const void* bias,
                int64_t m, int64_t k, int64_t n, const int64_t* rows, int64_t nrows,
                void* y, double* r, double* S) {
  if (op < OP_FWD || op > OP_DW || dt < DT_F32 || dt > DT_F16) return -1;
  if (m < 1 || k < 1 || n < 1 || !A || !B || !y) return -1;
  if (op != OP_FWD && bias) return -1;
  const int64_t out_rows = (op == OP_DW) ? k : m;
  const int64_t cols = (op == OP_DX) ? k : n;
  const int64_t L = (op == OP_FWD) ? k : (op == OP_DX ? n : m);  // reduction length
  if (!rows) nrows = out_rows;
  for (int64_t ii = 0; ii < nrows; ++ii) {
    const int64_t row = rows ? rows[ii] : ii;
    if (row < 0 || row >= out_rows) return -1;
  }

  // Operand sequences along the reduction index, upcast to float64:
  //   lhs(row)[l] and rhs(col)[l], l = 0 .. L-1.
  std::vector<double> rhs(static_cast<size_t>(cols * L));
  for (int64_t col = 0; col < cols; ++col) {
    for (int64_t l = 0; l < L; ++l) {
      int64_t idx;
      if (op == OP_FWD) idx = l * n + col;        // W[l, col]
      else if (op == OP_DX) idx = col * n + l;    // W[col, l]
      else idx = l * n + col;                     // dY[l, col]
      rhs[col * L + l] = decode(B, idx, dt);
    }
  }
  std::vector<double> lhs(static_cast<size_t>(L));
  for (int64_t ii = 0; ii < nrows; ++ii) {
    const int64_t row = rows ? rows[ii] : ii;
    for (int64_t l = 0; l < L; ++l) {
      int64_t idx;
      if (op == OP_FWD) idx = row * k + l;        // X[row, l]
      else if (op == OP_DX) idx = row * n + l;    // dY[row, l]
      else idx = l * k + row;                     // X[l, row]
      lhs[l] = decode(A, idx, dt);
    }
    for (int64_t col = 0; col < cols; ++col) {
      double abs_sum;
      double v = kbn_dot(lhs.data(), &rhs[col * L], L, &abs_sum);
      if (bias) {
        const double bj = decode(bias, col, dt);
        v = v + bj;
        abs_sum = abs_sum + std::fabs(bj);
      }
      const int64_t o = ii * cols + col;
      store(y, o, v, dt);
      if (r) r[o] = v;
      if (S) S[o] = abs_sum;
    }
  }
  return 0;
}


// ---- LayerNorm over the last dimension, float64 statistics ------------------
//
// Readings (the page gives only "float64 mean and variance"):
//   * every row sum is the matmul's tiled, compensated, fixed-order sum:
//     kbn_dot(v, ones) for a plain sum (fma(v, 1, p) = p + v, one rounding)
//     and kbn_dot(u, v) for a sum of products;
//   * mean = sum(x) / H; d_j = x_j - mean; var = sum(d_j * d_j) / H (the
//     biased variance, as a LayerNorm normalises); rstd = 1 / sqrt(var + eps);
//   * y_j = (d_j * rstd) * gamma_j + beta_j in float64, one rounding per
//     operation and no fusion; gamma or beta absent: that operation is
//     skipped; then one RNE rounding to the output dtype.
// Backward, with xhat_j = d_j * rstd (d_j recomputed from the stored mean) and
// g_j = dy_j * gamma_j (exact; g = dy without gamma):
//     a = sum(g) / H, b = sum(g_j * xhat_j) / H,
//     dx_j = rstd * ((g_j - a) - xhat_j * b)        then one rounding,
//     dgamma_j = sum over rows i of dy_ij * xhat_ij  (rows in tiles of 32, KBN),
//     dbeta_j  = sum over rows i of dy_ij            (the same column sum),
// which is the derivative of the forward's real-number definition.

namespace {

// mean, rstd and the float64 d_j of one row
void ln_stats(const void* x, int64_t row, int64_t h, double eps, int dt, std::vector<double>& d,
              double* mean, double* rstd) {
  std::vector<double> ones(static_cast<size_t>(h), 1.0);
  d.resize(static_cast<size_t>(h));
  for (int64_t j = 0; j < h; ++j) d[j] = decode(x, row * h + j, dt);
  double S;
  const double mu = kbn_dot(d.data(), ones.data(), h, &S) / static_cast<double>(h);
  for (int64_t j = 0; j < h; ++j) d[j] = d[j] - mu;
  const double var = kbn_dot(d.data(), d.data(), h, &S) / static_cast<double>(h);
  *mean = mu;
  *rstd = 1.0 / std::sqrt(var + eps);
}

}  // namespace

// Forward. x: rows x h in dt; gamma, beta: h in dt, nullable; y: rows x h in dt.
// mean, rstd: nullable float64[rows]; r: nullable float64 rows x h (y before rounding).
// Returns 0, or -1 on invalid arguments.
int oracle_layernorm_fwd(int dt, const void* x, const void* gamma, const void* beta, int64_t rows,
                         int64_t h, double eps, void* y, double* mean, double* rstd, double* r) {
  if (dt < DT_F32 || dt > DT_F16 || rows < 1 || h < 1 || !x || !y || !(eps >= 0.0)) return -1;
  std::vector<double> d;
  for (int64_t i = 0; i < rows; ++i) {
    double mu, rs;
    ln_stats(x, i, h, eps, dt, d, &mu, &rs);
    if (mean) mean[i] = mu;
    if (rstd) rstd[i] = rs;
    for (int64_t j = 0; j < h; ++j) {
      double v = d[j] * rs;
      if (gamma) v = v * decode(gamma, j, dt);
      if (beta) v = v + decode(beta, j, dt);
      store(y, i * h + j, v, dt);
      if (r) r[i * h + j] = v;
    }
  }
  return 0;
}

// Backward. dy, x: rows x h in dt; mean, rstd: float64[rows] from the forward;
// gamma: h in dt, nullable. dx: rows x h in dt (nullable); dgamma, dbeta: h in
// pdt (dt or f32), nullable; rdx: nullable float64 rows x h (dx before rounding).
int oracle_layernorm_bwd(int dt, int pdt, const void* dy, const void* x, const double* mean,
                         const double* rstd, const void* gamma, int64_t rows, int64_t h, void* dx,
                         void* dgamma, void* dbeta, double* rdx) {
  if (dt < DT_F32 || dt > DT_F16 || (pdt != dt && pdt != DT_F32)) return -1;
  if (rows < 1 || h < 1 || !dy || !x || !mean || !rstd) return -1;
  const double H = static_cast<double>(h);
  std::vector<double> xhat(static_cast<size_t>(h)), g(static_cast<size_t>(h));
  std::vector<double> ones(static_cast<size_t>(std::max(h, rows)), 1.0);
  std::vector<double> colx(static_cast<size_t>(rows * h)), coly(static_cast<size_t>(rows * h));
  for (int64_t i = 0; i < rows; ++i) {
    for (int64_t j = 0; j < h; ++j) {
      const double dyv = decode(dy, i * h + j, dt);
      xhat[j] = (decode(x, i * h + j, dt) - mean[i]) * rstd[i];
      g[j] = gamma ? dyv * decode(gamma, j, dt) : dyv;
      colx[j * rows + i] = xhat[j];   // column-major copies for the sums over rows
      coly[j * rows + i] = dyv;
    }
    if (!dx) continue;
    double S;
    const double a = kbn_dot(g.data(), ones.data(), h, &S) / H;
    const double b = kbn_dot(g.data(), xhat.data(), h, &S) / H;
    for (int64_t j = 0; j < h; ++j) {
      const double v = rstd[i] * ((g[j] - a) - xhat[j] * b);
      store(dx, i * h + j, v, dt);
      if (rdx) rdx[i * h + j] = v;
    }
  }
  for (int64_t j = 0; j < h; ++j) {
    double S;
    if (dgamma) store(dgamma, j, kbn_dot(&coly[j * rows], &colx[j * rows], rows, &S), pdt);
    if (dbeta) store(dbeta, j, kbn_dot(&coly[j * rows], ones.data(), rows, &S), pdt);
  }
  return 0;
}


// ---- correctly rounded tier -------------------------------------------------
//
// Carbon README (alia-carbon 0.2.0), "Roadmap", v0.2: the Kahan accumulation
// replaced by a superaccumulator, i.e. an exact sum whose value does not
// depend on the order of the terms. Reading taken: every output is the exact
// real value of sum_k a_k * b_k (+ b_j), rounded once to the output dtype with
// round-to-nearest-even (ties to the even code; beyond the largest finite
// value to infinity). An exact zero gives +0. If any term involves an infinity
// or a NaN, the result is the float64 sum of the terms (NaN or an infinity).
//
// The exact value is kept as a big integer: a sign and a magnitude in 32-bit
// limbs, counting units of 2^-BIG_LOW (below the lowest bit of any float64).
// Each float64 term m * 2^e (m an integer of at most 53 bits) is added to the
// positive or the negative magnitude at bit e + BIG_LOW; the two are
// subtracted at the end.

namespace {

constexpr int BIG_LOW = 1120;               // the unit is 2^-1120
constexpr int BIG_LIMBS = (BIG_LOW + 1100) / 32 + 2;

struct BigMag {
  std::vector<uint64_t> limb = std::vector<uint64_t>(BIG_LIMBS, 0);   // 32 bits used per limb
  void add_shifted(uint64_t m, int bit) {   // += m * 2^bit
    int li = bit / 32, sh = bit % 32;
    // m < 2^53: m << sh spans at most three 32-bit limbs
    unsigned __int128 v = static_cast<unsigned __int128>(m) << sh;
    uint64_t carry = 0;
    for (int i = li; i < BIG_LIMBS; ++i) {
      const uint64_t part = static_cast<uint64_t>(v & 0xffffffffu);
      v >>= 32;
      const uint64_t t = limb[i] + part + carry;
      limb[i] = t & 0xffffffffu;
      carry = t >> 32;
      if (v == 0 && carry == 0) break;
    }
  }
  int cmp(const BigMag& o) const {
    for (int i = BIG_LIMBS - 1; i >= 0; --i)
      if (limb[i] != o.limb[i]) return limb[i] < o.limb[i] ? -1 : 1;
    return 0;
  }
  void sub(const BigMag& o) {   // *this -= o, requires *this >= o
    int64_t borrow = 0;
    for (int i = 0; i < BIG_LIMBS; ++i) {
      int64_t t = static_cast<int64_t>(limb[i]) - static_cast<int64_t>(o.limb[i]) - borrow;
      borrow = t < 0 ? 1 : 0;
      if (t < 0) t += int64_t(1) << 32;
      limb[i] = static_cast<uint64_t>(t);
    }
  }
  int top_bit() const {   // index of the highest set bit, -1 for zero
    for (int i = BIG_LIMBS - 1; i >= 0; --i)
      if (limb[i]) return i * 32 + 63 - __builtin_clzll(limb[i]);
    return -1;
  }
  int bit(int b) const { return b < 0 ? 0 : static_cast<int>((limb[b / 32] >> (b % 32)) & 1u); }
  bool any_below(int b) const {   // any set bit with index < b
    for (int i = 0; i < b; ++i)
      if (bit(i)) return true;
    return false;
  }
};

struct ExactSum {
  BigMag pos, neg;
  double nonfinite = 0.0;
  bool has_nonfinite = false;
  void add(double v) {
    if (!std::isfinite(v)) {
      nonfinite = has_nonfinite ? nonfinite + v : v;
      has_nonfinite = true;
      return;
    }
    if (v == 0.0) return;
    int e;
    const double m = std::frexp(std::fabs(v), &e);            // |v| = m * 2^e, m in [0.5, 1)
    const uint64_t M = static_cast<uint64_t>(std::ldexp(m, 53));   // exact: 53-bit integer
    const int bit = e - 53 + BIG_LOW;                             // |v| = M * 2^(bit - BIG_LOW)
    (v > 0 ? pos : neg).add_shifted(M, bit);
  }
};

// Precision p (significand bits) and the exponent of the smallest normal value.
void dtype_format(int dt, int* p, int* emin) {
  if (dt == DT_F32) { *p = 24; *emin = -126; }
  else if (dt == DT_BF16) { *p = 8; *emin = -126; }
  else { *p = 11; *emin = -14; }
}

// The exact sum rounded once to dt (RNE), returned as a float64 that dt holds
// exactly (or an infinity past dt's range), then stored.
double round_exact(ExactSum& x, int dt) {
  if (x.has_nonfinite) return x.nonfinite;
  BigMag mag = x.pos;
  double sign = 1.0;
  const int c = x.pos.cmp(x.neg);
  if (c == 0) return 0.0;
  if (c > 0) {
    mag.sub(x.neg);
  } else {
    mag = x.neg;
    mag.sub(x.pos);
    sign = -1.0;
  }
  int p, emin;
  dtype_format(dt, &p, &emin);
  const int h = mag.top_bit();
  // the result's last bit: p - 1 bits below the top, but not below dt's smallest subnormal bit
  int lsb = h - (p - 1);
  const int lsb_min = (emin - (p - 1)) + BIG_LOW;
  if (lsb < lsb_min) lsb = lsb_min;
  uint64_t keep = 0;
  for (int b = h; b >= lsb; --b) keep = (keep << 1) | static_cast<uint64_t>(mag.bit(b));
  const int round = mag.bit(lsb - 1);
  const bool sticky = mag.any_below(lsb - 1);
  if (round && (sticky || (keep & 1u))) keep += 1;
  return sign * std::ldexp(static_cast<double>(keep), lsb - BIG_LOW);
}

}  // namespace

// Correctly rounded GEMM rows; arguments as oracle_gemm (no S).
int oracle_gemm_cr(int op, int dt, const void* A, const void* B, const void* bias,
                   int64_t m, int64_t k, int64_t n, const int64_t* rows, int64_t nrows, void* y) {
  if (op < OP_FWD || op > OP_DW || dt < DT_F32 || dt > DT_F16) return -1;
  if (m < 1 || k < 1 || n < 1 || !A || !B || !y) return -1;
  if (op != OP_FWD && bias) return -1;
  const int64_t out_rows = (op == OP_DW) ? k : m;
  const int64_t cols = (op == OP_DX) ? k : n;
  const int64_t L = (op == OP_FWD) ? k : (op == OP_DX ? n : m);
  if (!rows) nrows = out_rows;
  for (int64_t ii = 0; ii < nrows; ++ii) {
    const int64_t row = rows ? rows[ii] : ii;
    if (row < 0 || row >= out_rows) return -1;
  }
  for (int64_t ii = 0; ii < nrows; ++ii) {
    const int64_t row = rows ? rows[ii] : ii;
    for (int64_t col = 0; col < cols; ++col) {
      ExactSum x;
      for (int64_t l = 0; l < L; ++l) {
        double a, b;
        if (op == OP_FWD) { a = decode(A, row * k + l, dt); b = decode(B, l * n + col, dt); }
        else if (op == OP_DX) { a = decode(A, row * n + l, dt); b = decode(B, col * n + l, dt); }
        else { a = decode(A, l * k + row, dt); b = decode(B, l * n + col, dt); }
        x.add(a * b);   // exact: the product of two f32/bf16/f16 values fits float64
      }
      if (bias) x.add(decode(bias, col, dt));
      store(y, ii * cols + col, round_exact(x, dt), dt);
    }
  }
  return 0;
}

// The exact sum of cnt float64 values, rounded once to dt (pins the rounding of
// the correctly rounded tier on values chosen by the caller).
int oracle_exact_sum(const double* v, int64_t cnt, int dt, void* out) {
  if (dt < DT_F32 || dt > DT_F16 || cnt < 0 || (cnt > 0 && !v) || !out) return -1;
  ExactSum x;
  for (int64_t i = 0; i < cnt; ++i) x.add(v[i]);
  store(out, 0, round_exact(x, dt), dt);
  return 0;
}

}  // extern "C"

