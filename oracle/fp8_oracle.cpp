// CPU oracle for the block-scaled FP8 GEMM path.  TEST INFRASTRUCTURE ONLY.
//
// Only the test suite, the smoke check and the benchmark's CPU-baseline leg
// may load this library.  It shares no code, header or table with the GPU
// library: it is a plain, slow, obviously correct restatement of what the
// pages define, computed in FP64 and rounded once.
//
// Sources (cited by title and section):
//   [DG-day3]     "DeepSeek open-source week, day 3: DeepGEMM" (explinks.com):
//                 "Basic usage" example (operand and scale shapes, BF16 out),
//                 "Core features" (fine-grained scaling, two-level
//                 accumulation), "Source walk-through" part 3 (the promotion
//                 final += scale_a * scale_b * accum per 128-wide K block),
//                 and the three GEMM kinds (dense NT, contiguous-layout
//                 grouped, masked-layout grouped).
//   [GEMM-essay]  dpshk.com essay on GEMM and FP8 tuning (its headline is
//                 unrelated): §3.1 (E4M3 max about 448, min normal about
//                 2^-6), §3.3 ((A8*sA)x(B8*sB) = (A8xB8)*(sA*sB)).
//   [DG-usage]    kwkr.cn DeepGEMM usage article: §3.1 and the code in §4.2
//                 (scale = amax / 448, q = fp8(x / scale)).
//   [DG-practice] "DeepGEMM: FP8 GEMM kernel optimisation practice on Hopper
//                 Tensor Cores" (jianying88.com): §1.3 (A and B in E4M3 or
//                 E5M2, configurable), §3.1 (E4M3: 4 exponent / 3 mantissa
//                 bits, max about 448; E5M2: 5 / 2 bits, max about 57344),
//                 §5.2 (per-group scaling, 128 elements per group), §6.3-6.4
//                 (K tails).
//
// Readings where the pages are silent (each also listed in the design notes):
//   * FP8 is OCP E4M3FN: no infinities, NaN = S.1111.111, max 448; the second
//     format is OCP E5M2: infinities S.11111.00, NaN S.11111.xx (xx != 0),
//     max 57344.
//   * Encoding rounds to nearest, ties to even, and saturates at the format's
//     largest finite value (+-448, +-57344).
//   * A cast to E5M2 uses scale = amax / 57344, the rule amax / 448 with the
//     format's own maximum.
//   * An all-zero group or block gets scale 1.0f (codes all zero).
//   * The cast divides with IEEE fp32 correctly rounded division.
//   * K groups are [128g, 128g+128); the last one may be partial.  N blocks
//     likewise start at row 0.  Column j always uses the RHS scale of block
//     floor(j/128).
//   * The GEMM result is the plain dequantise-then-multiply definition; the
//     two-level accumulation reaches it up to FP32 rounding order, so the
//     oracle evaluates it in FP64 and rounds once to BF16 (nearest-even).
//   * Masked layout: counts are clamped to [0, max_m]; rows at or past the
//     count are not written.  Contiguous layout: a negative group index marks
//     a row that is not written.
//
// Logical scale layouts used here: LHS scales [rows][KG] row-major, RHS scales
// [NB][KG] row-major, KG = ceil(k/128), NB = ceil(n/128).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// ---- E4M3FN decode, closed form ([GEMM-essay] §3.1; OCP E4M3FN) ----------
// sign s, exponent e (4 bits, bias 7), mantissa f (3 bits).
//   e = 15, f = 7 : NaN
//   e = 0         : subnormal, f * 2^-9
//   otherwise     : (8 + f) * 2^(e - 10)   (= 1.f * 2^(e-7))
double e4m3_value(unsigned code) {
  const unsigned s = (code >> 7) & 1u, e = (code >> 3) & 15u, f = code & 7u;
  if (e == 15u && f == 7u) return std::nan("");
  const double mag = (e == 0u) ? std::ldexp(double(f), -9)
                               : std::ldexp(double(8u + f), int(e) - 10);
  return s ? -mag : mag;
}

// ---- E5M2 decode, closed form ([DG-practice] §3.1; OCP E5M2) ---------------
// sign s, exponent e (5 bits, bias 15), mantissa f (2 bits).
//   e = 31, f = 0 : infinity;  e = 31, f != 0 : NaN
//   e = 0         : subnormal, f * 2^-16
//   otherwise     : (4 + f) * 2^(e - 17)   (= 1.f * 2^(e-15))
double e5m2_value(unsigned code) {
  const unsigned s = (code >> 7) & 1u, e = (code >> 2) & 31u, f = code & 3u;
  double mag;
  if (e == 31u) mag = f == 0u ? HUGE_VAL : std::nan("");
  else mag = (e == 0u) ? std::ldexp(double(f), -16) : std::ldexp(double(4u + f), int(e) - 17);
  return s ? -mag : mag;
}

// Formats: 0 = E4M3FN, 1 = E5M2.
constexpr int kE4M3 = 0, kE5M2 = 1;

struct Table {
  double v[256];
  uint8_t max_code;  // largest finite non-negative code
  explicit Table(int fmt) {
    for (unsigned c = 0; c < 256; ++c) v[c] = fmt == kE5M2 ? e5m2_value(c) : e4m3_value(c);
    max_code = fmt == kE5M2 ? 0x7B : 0x7E;
  }
};
const Table& table(int fmt = kE4M3) {
  static const Table t4(kE4M3), t5(kE5M2);
  return fmt == kE5M2 ? t5 : t4;
}

// ---- encode: nearest finite magnitude, ties to even, saturating ------------
// The non-negative finite codes 0x00..max_code are strictly increasing in
// value (both formats), so the nearest one is found by bisection on that
// sorted list.  NaN encodes as 0x7F (a NaN in both formats).
uint8_t fp8_encode(double x, int fmt) {
  if (std::isnan(x)) return 0x7F;
  const uint8_t sign = std::signbit(x) ? 0x80 : 0x00;
  const double a = std::fabs(x);
  const Table& tb = table(fmt);
  const double* v = tb.v;
  if (a >= v[tb.max_code]) return uint8_t(sign | tb.max_code);
  // largest code lo with v[lo] <= a  (v[0] = 0 <= a always holds)
  int lo = 0, hi = tb.max_code;
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (v[mid] <= a) lo = mid; else hi = mid;
  }
  int c = lo;
  if (v[lo] != a) {
    const double dlo = a - v[lo], dhi = v[hi] - a;
    if (dhi < dlo || (dhi == dlo && (hi & 1) == 0)) c = hi;
  }
  return uint8_t(sign | c);
}
uint8_t e4m3_encode(double x) { return fp8_encode(x, kE4M3); }

// ---- BF16 round-to-nearest-even, straight from double ----------------------
// Keeps 8 significant bits (quantum 2^(e-8) for a in [2^(e-1), 2^e)); below
// the normal range the quantum is the subnormal step 2^-133.  Rounding from
// double directly avoids a double rounding through fp32.
uint16_t bf16_from_double(double x) {
  if (std::isnan(x)) return 0x7FC0;
  const uint16_t sign = std::signbit(x) ? 0x8000 : 0x0000;
  const double a = std::fabs(x);
  if (a == 0.0) return sign;
  if (std::isinf(a)) return uint16_t(sign | 0x7F80);
  int e = 0;
  std::frexp(a, &e);
  const int qexp = std::max(e - 8, -133);
  const double r = std::nearbyint(std::ldexp(a, -qexp));  // ties to even
  const double v = std::ldexp(r, qexp);
  const double max_finite = std::ldexp(255.0, 120);        // 0x7F7F
  if (v > max_finite) return uint16_t(sign | 0x7F80);
  const float fv = float(v);  // exact: v has at most 8 significant bits
  uint32_t u;
  std::memcpy(&u, &fv, 4);
  return uint16_t(sign | (u >> 16));
}

template <class F>
void parallel_rows(int64_t rows, int nthreads, F&& body) {
  if (nthreads <= 1 || rows < 2) { body(int64_t(0), rows); return; }
  const int64_t t = std::min<int64_t>(nthreads, rows);
  std::vector<std::thread> pool;
  for (int64_t w = 0; w < t; ++w) {
    const int64_t r0 = rows * w / t, r1 = rows * (w + 1) / t;
    pool.emplace_back([=, &body] { body(r0, r1); });
  }
  for (auto& th : pool) th.join();
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- integer form of the codes --------------------------------------------
// Every finite E4M3 value is an integer multiple of 2^-9 (the smallest
// subnormal) and every finite E5M2 value a multiple of 2^-16, so code c has
// value mant[c] * 2^-q with an integer mant[c] (|mant| <= 448 * 2^9 for E4M3,
// <= 57344 * 2^16 < 2^32 for E5M2).  nonfinite[c] marks NaN / infinity codes.
struct IntTable {
  int64_t mant[256];
  uint8_t nonfinite[256];
  int q;
  explicit IntTable(int fmt) {
    q = fmt == kE5M2 ? 16 : 9;
    for (unsigned c = 0; c < 256; ++c) {
      const double v = table(fmt).v[c];
      nonfinite[c] = std::isfinite(v) ? 0 : 1;
      mant[c] = std::isfinite(v) ? int64_t(std::ldexp(v, q)) : 0;  // exact
    }
  }
};
const IntTable& int_table(int fmt) {
  static const IntTable t4(kE4M3), t5(kE5M2);
  return fmt == kE5M2 ? t5 : t4;
}

// ---- one output element of the block-scaled GEMM ---------------------------
// [DG-day3] "Core features" and "Source walk-through" part 3:
//   D[i][j] = sum_g (sa[i][g] * sb[j/128][g]) * S_g(i, j),
//   S_g(i, j) = sum_{t in K group g} dec(A[i][t]) * dec(B[j][t]).
// S_g is summed exactly on the integer mantissas (a 128-term sum of products
// below 2^64 each fits in 128 bits) and rounded once to FP64.  For two E4M3
// operands that rounding is exact: the sum is an integer below 2^43 times
// 2^-18.  With an E5M2 operand the exact sum can need up to about 71
// significant bits (products are multiples of 2^-32 up to 2^31.6), so S_g is
// the correctly rounded FP64 value of the exact sum.  A NaN or infinite code
// in the group makes S_g the plain FP64 sum of the decoded products, so the
// NaN or infinity propagates as IEEE arithmetic gives it.
double group_sum(const uint8_t* a, const uint8_t* b, int64_t len, int a_fmt, int b_fmt) {
  const IntTable& ia = int_table(a_fmt);
  const IntTable& ib = int_table(b_fmt);
  __int128 s = 0;
  unsigned bad = 0;
  for (int64_t t = 0; t < len; ++t) {
    s += __int128(ia.mant[a[t]]) * __int128(ib.mant[b[t]]);
    bad |= unsigned(ia.nonfinite[a[t]] | ib.nonfinite[b[t]]);
  }
  if (!bad) return std::ldexp(double(s), -(ia.q + ib.q));  // one rounding (int128 -> double is RNE)
  const double* va = table(a_fmt).v;
  const double* vb = table(b_fmt).v;
  double d = 0.0;
  for (int64_t t = 0; t < len; ++t) d += va[a[t]] * vb[b[t]];
  return d;
}

double gemm_element(const uint8_t* a_row, const float* sa_row,
                    const uint8_t* b_row, const float* sb_row, int64_t k,
                    int a_fmt = kE4M3, int b_fmt = kE4M3) {
  const int64_t kg = ceil_div(k, 128);
  double acc = 0.0;
  for (int64_t g = 0; g < kg; ++g) {
    const int64_t t0 = g * 128, t1 = std::min<int64_t>(t0 + 128, k);
    const double s = group_sum(a_row + t0, b_row + t0, t1 - t0, a_fmt, b_fmt);
    acc += (double(sa_row[g]) * double(sb_row[g])) * s;
  }
  return acc;
}

// Rows [r0, r1) of D = A . B^T with one RHS (B, sb) for every row.
void gemm_rows(const uint8_t* A, const float* sa, const uint8_t* B,
               const float* sb, int64_t n, int64_t k, int64_t r0, int64_t r1,
               uint16_t* out, double* pre, int a_fmt = kE4M3, int b_fmt = kE4M3) {
  const int64_t kg = ceil_div(k, 128);
  for (int64_t i = r0; i < r1; ++i)
    for (int64_t j = 0; j < n; ++j) {
      const double d = gemm_element(A + i * k, sa + i * kg, B + j * k,
                                    sb + (j / 128) * kg, k, a_fmt, b_fmt);
      out[i * n + j] = bf16_from_double(d);
      if (pre) pre[i * n + j] = d;
    }
}

// Per-group amax -> scale -> codes, for one group of `len` elements spread
// with stride `stride` ([DG-usage] §3.1/§4.2; [DG-practice] §5.2).
float group_scale(float amax, int fmt = kE4M3) {
  if (amax == 0.0f) return 1.0f;  // reading: an all-zero group keeps codes 0
  return amax / (fmt == kE5M2 ? 57344.0f : 448.0f);  // IEEE fp32, correctly rounded
}

}  // namespace

extern "C" {

// Value of every E4M3FN code (NaN for 0x7F and 0xFF).
void orc_e4m3_table(double* out256) {
  for (int c = 0; c < 256; ++c) out256[c] = table().v[c];
}

uint8_t orc_e4m3_encode(double x) { return e4m3_encode(x); }

void orc_e4m3_encode_array(const double* x, int64_t count, uint8_t* q) {
  for (int64_t i = 0; i < count; ++i) q[i] = e4m3_encode(x[i]);
}

// The same two for either format (0 = E4M3FN, 1 = E5M2).
void orc_fp8_table(int fmt, double* out256) {
  for (int c = 0; c < 256; ++c) out256[c] = table(fmt).v[c];
}
void orc_fp8_encode_array(int fmt, const double* x, int64_t count, uint8_t* q) {
  for (int64_t i = 0; i < count; ++i) q[i] = fp8_encode(x[i], fmt);
}

uint16_t orc_bf16_rne(double x) { return bf16_from_double(x); }

void orc_bf16_rne_array(const double* x, int64_t count, uint16_t* out) {
  for (int64_t i = 0; i < count; ++i) out[i] = bf16_from_double(x[i]);
}

// Per-token-group cast of an fp32 [m][k] matrix: one scale per row and per
// 128-wide K group.  q [m][k] codes, scales [m][KG] (logical layout).
void orc_cast_1x128_f32(const float* x, int64_t m, int64_t k, uint8_t* q,
                        float* scales, int nthreads, int fmt) {
  const int64_t kg = ceil_div(k, 128);
  parallel_rows(m, nthreads, [&](int64_t r0, int64_t r1) {
    for (int64_t i = r0; i < r1; ++i)
      for (int64_t g = 0; g < kg; ++g) {
        const int64_t t0 = g * 128, t1 = std::min<int64_t>(t0 + 128, k);
        float amax = 0.0f;
        for (int64_t t = t0; t < t1; ++t) amax = std::max(amax, std::fabs(x[i * k + t]));
        const float s = group_scale(amax, fmt);
        scales[i * kg + g] = s;
        for (int64_t t = t0; t < t1; ++t) {
          const float y = x[i * k + t] / s;
          q[i * k + t] = fp8_encode(double(y), fmt);
        }
      }
  });
}

// Same, for bf16 input (bit patterns); each value widens exactly to fp32.
void orc_cast_1x128_bf16(const uint16_t* x, int64_t m, int64_t k, uint8_t* q,
                         float* scales, int nthreads, int fmt) {
  std::vector<float> xf(size_t(m * k));
  for (int64_t i = 0; i < m * k; ++i) {
    const uint32_t u = uint32_t(x[i]) << 16;
    std::memcpy(&xf[size_t(i)], &u, 4);
  }
  orc_cast_1x128_f32(xf.data(), m, k, q, scales, nthreads, fmt);
}

// Block cast of an fp32 [n][k] weight: one scale per 128x128 block, the
// edge blocks using only their real elements.  scales [NB][KG].
void orc_cast_128x128_f32(const float* w, int64_t n, int64_t k, uint8_t* q,
                          float* scales, int nthreads, int fmt) {
  const int64_t kg = ceil_div(k, 128), nb = ceil_div(n, 128);
  parallel_rows(nb, nthreads, [&](int64_t b0, int64_t b1) {
    for (int64_t b = b0; b < b1; ++b)
      for (int64_t g = 0; g < kg; ++g) {
        const int64_t i0 = b * 128, i1 = std::min<int64_t>(i0 + 128, n);
        const int64_t t0 = g * 128, t1 = std::min<int64_t>(t0 + 128, k);
        float amax = 0.0f;
        for (int64_t i = i0; i < i1; ++i)
          for (int64_t t = t0; t < t1; ++t) amax = std::max(amax, std::fabs(w[i * k + t]));
        const float s = group_scale(amax, fmt);
        scales[b * kg + g] = s;
        for (int64_t i = i0; i < i1; ++i)
          for (int64_t t = t0; t < t1; ++t) {
            const float y = w[i * k + t] / s;
            q[i * k + t] = fp8_encode(double(y), fmt);
          }
      }
  });
}

// Dense NT GEMM: A [m][k], sa [m][KG], B [n][k], sb [NB][KG] -> out [m][n]
// bf16 bits.  `pre` (optional, [m][n]) receives the FP64 value before the
// BF16 rounding.
// a_fmt / b_fmt: the operands' formats (0 = E4M3FN, 1 = E5M2).
void orc_gemm_nt(const uint8_t* A, const float* sa, const uint8_t* B,
                 const float* sb, int64_t m, int64_t n, int64_t k,
                 uint16_t* out, double* pre, int nthreads, int a_fmt, int b_fmt) {
  parallel_rows(m, nthreads, [&](int64_t r0, int64_t r1) {
    gemm_rows(A, sa, B, sb, n, k, r0, r1, out, pre, a_fmt, b_fmt);
  });
}

// Contiguous-layout grouped GEMM ([DG-day3], the M-axis grouped kind):
// A [M][k], sa [M][KG], B [G][n][k], sb [G][NB][KG], m_indices [M].
// Row i uses group m_indices[i]; a negative index leaves row i untouched.
void orc_gemm_contiguous(const uint8_t* A, const float* sa, const uint8_t* B,
                         const float* sb, const int32_t* m_indices,
                         int64_t m_total, int64_t n, int64_t k, int64_t groups,
                         uint16_t* out, double* pre, int nthreads) {
  const int64_t kg = ceil_div(k, 128), nb = ceil_div(n, 128);
  parallel_rows(m_total, nthreads, [&](int64_t r0, int64_t r1) {
    for (int64_t i = r0; i < r1; ++i) {
      const int64_t g = m_indices[i];
      if (g < 0 || g >= groups) continue;
      gemm_rows(A, sa, B + g * n * k, sb + g * nb * kg, n, k, i, i + 1, out,
                pre);
    }
  });
}

// Masked-layout grouped GEMM ([DG-day3], the masked kind):
// A [G][max_m][k], sa [G][max_m][KG], B [G][n][k], sb [G][NB][KG],
// masked_m [G]; out [G][max_m][n].  Rows r < clamp(masked_m[g], 0, max_m)
// of group g are computed; every other row is left untouched.
void orc_gemm_masked(const uint8_t* A, const float* sa, const uint8_t* B,
                     const float* sb, const int32_t* masked_m, int64_t groups,
                     int64_t max_m, int64_t n, int64_t k, uint16_t* out,
                     double* pre, int nthreads) {
  const int64_t kg = ceil_div(k, 128), nb = ceil_div(n, 128);
  for (int64_t g = 0; g < groups; ++g) {
    const int64_t cnt = std::min<int64_t>(std::max<int64_t>(masked_m[g], 0), max_m);
    const uint8_t* Ag = A + g * max_m * k;
    const float* sag = sa + g * max_m * kg;
    uint16_t* og = out + g * max_m * n;
    double* pg = pre ? pre + g * max_m * n : nullptr;
    parallel_rows(cnt, nthreads, [&](int64_t r0, int64_t r1) {
      gemm_rows(Ag, sag, B + g * n * k, sb + g * nb * kg, n, k, r0, r1, og, pg);
    });
  }
}

// Selected elements of D = A . B^T for one RHS: for each p, the element
// (rows[p], cols[p]); A rows are indexed directly ([*][k], sa [*][KG]).
void orc_gemm_points(const uint8_t* A, const float* sa, const uint8_t* B,
                     const float* sb, int64_t k, const int64_t* rows,
                     const int64_t* cols, int64_t npts, uint16_t* out,
                     double* pre, int nthreads, int a_fmt, int b_fmt) {
  const int64_t kg = ceil_div(k, 128);
  parallel_rows(npts, nthreads, [&](int64_t p0, int64_t p1) {
    for (int64_t p = p0; p < p1; ++p) {
      const int64_t i = rows[p], j = cols[p];
      const double d = gemm_element(A + i * k, sa + i * kg, B + j * k,
                                    sb + (j / 128) * kg, k, a_fmt, b_fmt);
      out[p] = bf16_from_double(d);
      if (pre) pre[p] = d;
    }
  });
}

int orc_hardware_threads(void) {
  const unsigned t = std::thread::hardware_concurrency();
  return t ? int(t) : 1;
}

}  // extern "C"
