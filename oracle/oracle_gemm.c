/*
 * Oracle for the dense bf16 GEMM  C[M,N] = A[M,K] * B[N,K]^T.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct CPU
 * definition that the GPU library is checked against.  Only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product library never links, calls or falls back to it, and the two share
 * no source.
 *
 * What it computes (the plain definition of the operation):
 *
 *   - Page "Matrix Multiplication on NVIDIA's Blackwell: A Four-Part Deep
 *     Dive", section on the definition of matrix multiplication: C is the
 *     set of M x N inner products over the K dimension, written as a triple
 *     loop over row, column and inner index.
 *   - Same page, section "naive kernel (Kernel 1) and data types": the
 *     second operand is indexed b[col, k] (stored N x K, K contiguous), the
 *     inputs and output are bf16, and the sum is carried in a wider type
 *     than bf16.  Here the sum is carried in fp64, in natural k order, so
 *     it is exact for every input this project draws from (bf16 x bf16
 *     products are exact in fp64, and the integer-valued sets stay far
 *     below 2^53).
 *   - Page "Hand-writing a Blackwell GEMM: from 164 to 1400 TFLOP/s",
 *     section "Step 1: the K loop": a tile of C is the sum over K-slices
 *     of A_k B_k^T, starting from zero.  That sum is the same number as the
 *     triple loop, which is what this file evaluates.
 *
 * Readings where the pages are silent:
 *   - The fp64 sum is rounded to bf16 once, directly, with IEEE
 *     round-to-nearest-even (no detour through fp32, so no double
 *     rounding).
 *   - K = 0 gives the empty sum, 0.
 *   - bf16 subnormal results are produced by clamping the quantum at 2^-133;
 *     overflow past the largest finite bf16 gives +-infinity.
 *
 *   - The fp16-input variant (same page, measurement section: the
 *     comparisons run on fp16 tensors) is the same sum over fp16 operands,
 *     rounded once to fp16: IEEE binary16, round to nearest even,
 *     subnormals down to 2^-24, overflow past 65504 to +-infinity.
 *
 * Layouts (strides in elements):
 *   A(m,k) = A[m*lda + k], B(n,k) = B[n*ldb + k], C(m,n) = C[m*ldc + n].
 *   bf16 and fp16 values are passed as their raw 16-bit patterns (uint16_t).
 *
 * Parallelism: rows of C are split across OpenMP threads.  Each element is
 * still computed by one plain loop over k, so the result does not depend on
 * the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 bit pattern -> double.  A bf16 is the top half of an IEEE binary32,
 * so the decode is exact. */
static double bf16_bits_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* double -> bf16 bit pattern, round to nearest, ties to even, in one step.
 *
 * bf16 keeps 8 significant bits (1 implicit + 7 stored), exponent range as
 * binary32: normal numbers from 2^-126, subnormals down to 2^-133.  For
 * x = f * 2^e with 0.5 <= |f| < 1, the spacing of bf16 values around x is
 * 2^(e-8), but never finer than the subnormal spacing 2^-133.  Scaling x by
 * that spacing, rounding to an integer with ties to even (nearbyint in the
 * default rounding mode), and scaling back gives the nearest bf16 value; all
 * scalings are by powers of two and therefore exact. */
uint16_t oracle_round_f64_to_bf16(double x) {
  if (isnan(x)) return 0x7FC0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  if (isinf(x)) return sign | 0x7F80;
  if (x == 0.0) return sign;
  int e;
  (void)frexp(x, &e);
  int q = e - 8;
  if (q < -133) q = -133;
  double r = ldexp(nearbyint(ldexp(x, -q)), q);
  /* largest finite bf16 is (2 - 2^-7) * 2^127 */
  if (fabs(r) > 0x1.fep127) return sign | 0x7F80;
  if (r == 0.0) return sign;
  float f = (float)r; /* exact: r is a bf16 value */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

/* fp16 bit pattern -> double, from the IEEE 754 binary16 layout: sign bit,
 * 5 exponent bits with bias 15, 10 fraction bits.  Exponent field 0 holds
 * zero and the subnormals f * 2^-24; field 31 holds infinity and NaN;
 * otherwise the value is (1024 + f) * 2^(e - 25).  Exact in double. */
double oracle_f16_bits_to_f64(uint16_t h) {
  const int e = (h >> 10) & 31, f = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25);
  return (h & 0x8000) ? -v : v;
}

/* double -> fp16 bit pattern, round to nearest, ties to even, in one step.
 *
 * fp16 keeps 11 significant bits; normal numbers start at 2^-14 and the
 * subnormal spacing is 2^-24.  As for bf16: with x = f * 2^e, 0.5 <= |f| < 1,
 * the spacing around x is 2^(e-11), clamped below at 2^-24; round x / spacing
 * to an integer (ties to even) and scale back.  The largest finite value is
 * (2 - 2^-10) * 2^15 = 65504; a rounded result beyond it is infinite. */
uint16_t oracle_round_f64_to_f16(double x) {
  if (isnan(x)) return 0x7E00;
  const uint16_t sign = signbit(x) ? 0x8000 : 0;
  if (isinf(x)) return sign | 0x7C00;
  if (x == 0.0) return sign;
  int e;
  (void)frexp(x, &e);
  int q = e - 11;
  if (q < -24) q = -24;
  const double r = fabs(ldexp(nearbyint(ldexp(x, -q)), q));
  if (r > 65504.0) return sign | 0x7C00;
  if (r == 0.0) return sign;
  /* encode the exact fp16 value r */
  int re;
  const double rf = frexp(r, &re); /* r = rf * 2^re, 0.5 <= rf < 1 */
  if (re - 1 < -14) /* subnormal: r = f * 2^-24 with f < 1024 */
    return sign | (uint16_t)ldexp(r, 24);
  const int field = re - 1 + 15;                      /* biased exponent */
  const int frac = (int)ldexp(rf, 11) - 1024;         /* 10 stored bits */
  return sign | (uint16_t)(field << 10) | (uint16_t)frac;
}

typedef uint16_t (*round_fn)(double);

/* One element: s = sum_k A(m,k) * B(n,k) in fp64, k ascending; operands
 * decoded as fp16 when half != 0, else as bf16.  (One loop per format, so
 * the decode is inlined into it.) */
static double dot_f64(int half, const uint16_t* a_row, const uint16_t* b_row, int64_t K) {
  double s = 0.0;
  if (half) {
    for (int64_t k = 0; k < K; ++k)
      s += oracle_f16_bits_to_f64(a_row[k]) * oracle_f16_bits_to_f64(b_row[k]);
  } else {
    for (int64_t k = 0; k < K; ++k)
      s += bf16_bits_to_f64(a_row[k]) * bf16_bits_to_f64(b_row[k]);
  }
  return s;
}

static int gemm_any(int half, round_fn rnd, int64_t M, int64_t N, int64_t K,
                    const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                    uint16_t* C, int64_t ldc, double* S, int64_t lds, int nthreads) {
  if (M < 0 || N < 0 || K < 0) return -1;
  if (lda < K || ldb < K) return -1;
  if (C && ldc < N) return -1;
  if (S && lds < N) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t n = 0; n < N; ++n) {
      double s = dot_f64(half, A + m * lda, B + n * ldb, K);
      if (C) C[m * ldc + n] = rnd(s);
      if (S) S[m * lds + n] = s;
    }
  }
  (void)nthreads;
  return 0;
}

static int entries_any(int half, round_fn rnd, int64_t M, int64_t N, int64_t K,
                       const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                       int64_t count, const int64_t* ms, const int64_t* ns,
                       uint16_t* out16, double* out_f64, int nthreads) {
  if (M < 0 || N < 0 || K < 0 || count < 0) return -1;
  if (lda < K || ldb < K) return -1;
  for (int64_t i = 0; i < count; ++i)
    if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
  for (int64_t i = 0; i < count; ++i) {
    double s = dot_f64(half, A + ms[i] * lda, B + ns[i] * ldb, K);
    if (out16) out16[i] = rnd(s);
    if (out_f64) out_f64[i] = s;
  }
  (void)nthreads;
  return 0;
}

/* Full GEMM.  C (bf16, stride ldc) and S (fp64 sums, stride lds) are each
 * optional (NULL to skip).  nthreads <= 0 lets OpenMP choose.
 * Returns 0, or -1 on a malformed argument. */
int oracle_gemm_bf16(int64_t M, int64_t N, int64_t K,
                     const uint16_t* A, int64_t lda,
                     const uint16_t* B, int64_t ldb,
                     uint16_t* C, int64_t ldc,
                     double* S, int64_t lds,
                     int nthreads) {
  return gemm_any(0, oracle_round_f64_to_bf16, M, N, K, A, lda, B, ldb, C,
                  ldc, S, lds, nthreads);
}

/* The same product over fp16 operands, C rounded to fp16. */
int oracle_gemm_f16(int64_t M, int64_t N, int64_t K,
                    const uint16_t* A, int64_t lda,
                    const uint16_t* B, int64_t ldb,
                    uint16_t* C, int64_t ldc,
                    double* S, int64_t lds,
                    int nthreads) {
  return gemm_any(1, oracle_round_f64_to_f16, M, N, K, A, lda, B, ldb,
                  C, ldc, S, lds, nthreads);
}

/* Listed elements only: for i < count, element (ms[i], ns[i]) of the same
 * product.  Used where the full product is too large to evaluate on the
 * host in test time.  out16 / out_f64 are each optional. */
int oracle_gemm_bf16_entries(int64_t M, int64_t N, int64_t K,
                             const uint16_t* A, int64_t lda,
                             const uint16_t* B, int64_t ldb,
                             int64_t count, const int64_t* ms, const int64_t* ns,
                             uint16_t* out16, double* out_f64,
                             int nthreads) {
  return entries_any(0, oracle_round_f64_to_bf16, M, N, K, A, lda, B, ldb,
                     count, ms, ns, out16, out_f64, nthreads);
}

int oracle_gemm_f16_entries(int64_t M, int64_t N, int64_t K,
                            const uint16_t* A, int64_t lda,
                            const uint16_t* B, int64_t ldb,
                            int64_t count, const int64_t* ms, const int64_t* ns,
                            uint16_t* out16, double* out_f64,
                            int nthreads) {
  return entries_any(1, oracle_round_f64_to_f16, M, N, K, A, lda, B,
                     ldb, count, ms, ns, out16, out_f64, nthreads);
}

/* Threads OpenMP would use (for reporting the CPU baseline honestly). */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
