/*
 * oracle.c -- plain CPU reference for the tiled dense GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or helper with the
 * HIP kernels.
 *
 * What it computes (the plain definition the tiled kernels reach faster):
 *
 *   "TIRx GEMM on Blackwell", section "The short version": the operation is
 *   D = A @ B.T with FP16 inputs and output and FP32 accumulation.
 *   TileFoundry "Choosing schedules and instructions for a backend",
 *   section 1 (the GRID HIR): a is (M, K), b is (K, N), the accumulator
 *   starts at zero, each K block adds matmul(a_tile, b_tile) in f32, and the
 *   accumulator is cast to bf16 once at the end.
 *   CMU "TIRx" blog, section "Why we built TIRx": each output element is the
 *   dot product of a row of A and a column of B.
 *
 * So for i < M, j < N:
 *     d[i][j] = sum_{k=0}^{K-1} a[i][k] * bhat[k][j]
 *     s[i][j] = sum_{k=0}^{K-1} |a[i][k] * bhat[k][j]|
 * with bhat[k][j] = B[j*ldb + k] for the A.B^T ("NT") layout and
 * bhat[k][j] = B[k*ldb + j] for the A.B ("NN") layout, both row-major as in
 * the conventional layout rule of the CMU blog (offset = row*stride + col).
 *
 * Inputs are FP16 or BF16 bit patterns, widened exactly to double.  Every
 * product of two such values is exact in double (at most 22 significant
 * bits), and the sum is taken in double in ascending k.  The result is
 * rounded to the output format once, directly from double, with IEEE
 * round-to-nearest-even (overflow to infinity): that is the plainest reading
 * of the pages' single "cast" of the accumulator.
 *
 * The acceptance test lives here too: an element passes when
 *     |d_gpu - d| <= ulp_out(|d|) + 2^-11 * s,
 * where ulp_out(x) is the spacing of the output format at x (the smallest
 * subnormal for x below the normal range).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_FMT_F16 0
#define ORACLE_FMT_BF16 1
#define ORACLE_NT 0
#define ORACLE_NN 1

/* ---- format parameters (IEEE 754 binary16; bfloat16) -------------------- */
/* precision p (significant bits incl. the hidden one), minimum normal
 * exponent emin, exponent bias, fraction-field width. */
static int fmt_p(int fmt) { return fmt == ORACLE_FMT_F16 ? 11 : 8; }
static int fmt_emin(int fmt) { return fmt == ORACLE_FMT_F16 ? -14 : -126; }
static int fmt_emax(int fmt) { return fmt == ORACLE_FMT_F16 ? 15 : 127; }
static int fmt_bias(int fmt) { return fmt == ORACLE_FMT_F16 ? 15 : 127; }
static int fmt_expbits(int fmt) { return fmt == ORACLE_FMT_F16 ? 5 : 8; }

/* Decode a 16-bit pattern of the given format to its exact double value. */
double oracle_decode(int fmt, uint16_t bits) {
  int fbits = fmt_p(fmt) - 1;
  int ebits = fmt_expbits(fmt);
  int sign = (bits >> 15) & 1;
  int e = (bits >> fbits) & ((1 << ebits) - 1);
  int f = bits & ((1 << fbits) - 1);
  double v;
  if (e == 0) {
    /* subnormal or zero: f * 2^(emin - fbits) */
    v = ldexp((double)f, fmt_emin(fmt) - fbits);
  } else if (e == (1 << ebits) - 1) {
    v = f ? NAN : INFINITY;
  } else {
    /* normal: (2^fbits + f) * 2^(e - bias - fbits) */
    v = ldexp((double)((1 << fbits) + f), e - fmt_bias(fmt) - fbits);
  }
  return sign ? -v : v;
}

/* Round a double to the nearest representable value of the format, ties to
 * even, overflow to infinity; return the bit pattern. */
uint16_t oracle_round(int fmt, double x) {
  int p = fmt_p(fmt), fbits = p - 1;
  int emin = fmt_emin(fmt), emax = fmt_emax(fmt);
  if (isnan(x)) return (uint16_t)(0x7fff & ~((1 << (fbits - 1)) - 1)); /* quiet NaN */
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  uint16_t inf = (uint16_t)(((1 << fmt_expbits(fmt)) - 1) << fbits);
  if (isinf(a)) return sign | inf;
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2);          /* a = m * 2^e2 with m in [0.5, 1) */
  int E = e2 - 1;         /* floor(log2 a) */
  if (E < emin) E = emin; /* below the normal range the spacing is fixed */
  double q = ldexp(1.0, E - fbits); /* spacing of the format in this binade */
  /* a / q and r * q only move the exponent, so they are exact; nearbyint
   * uses the default rounding direction, round-half-even. */
  double r = nearbyint(a / q) * q;
  if (r >= ldexp(1.0, emax + 1)) return sign | inf;
  if (r == 0.0) return sign;
  /* encode r exactly */
  frexp(r, &e2);
  int Er = e2 - 1;
  if (Er < emin) {
    /* subnormal: r = f * 2^(emin - fbits) */
    uint16_t f = (uint16_t)ldexp(r, -(emin - fbits));
    return sign | f;
  }
  uint16_t f = (uint16_t)(ldexp(r, -(Er - fbits)) - (double)(1 << fbits));
  uint16_t e = (uint16_t)(Er + fmt_bias(fmt));
  return sign | (uint16_t)(e << fbits) | f;
}

/* Spacing of the output format at |x|: 2^(max(floor(log2|x|), emin) - p + 1);
 * at zero it is the smallest subnormal. */
double oracle_ulp(int fmt, double x) {
  double a = fabs(x);
  int E;
  if (a == 0.0 || !isfinite(a)) {
    E = fmt_emin(fmt);
  } else {
    int e2;
    frexp(a, &e2);
    E = e2 - 1;
    if (E < fmt_emin(fmt)) E = fmt_emin(fmt);
  }
  return ldexp(1.0, E - fmt_p(fmt) + 1);
}

/* One output element: the ascending-k dot product and its absolute sum. */
static void dot_one(int layout, int fmt, int64_t K, const uint16_t* A, int64_t lda,
                    const uint16_t* B, int64_t ldb, int64_t i, int64_t j,
                    double* d_out, double* s_out) {
  double d = 0.0, s = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    double a = oracle_decode(fmt, A[i * lda + k]);
    double b = (layout == ORACLE_NT) ? oracle_decode(fmt, B[j * ldb + k])
                                     : oracle_decode(fmt, B[k * ldb + j]);
    double prod = a * b; /* exact */
    d += prod;
    s += fabs(prod);
  }
  *d_out = d;
  *s_out = s;
}

/* Full product.  D and S are M x N row-major with leading dimension ldo
 * (either may be NULL).  A and B are first widened to double: a64[i][k] and
 * bt64[j][k] = bhat[k][j] (the second operand stored one column per row, so
 * the inner loop reads both contiguously).  Rows are split over OpenMP
 * threads; each element is still the same ascending-k sum.  Returns 0, or -1
 * if the scratch arrays cannot be allocated. */
int oracle_gemm(int layout, int fmt, int64_t M, int64_t N, int64_t K,
                const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                double* D, double* S, int64_t ldo) {
  double* a64 = (double*)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
  double* bt64 = (double*)malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
  if (!a64 || !bt64) {
    free(a64);
    free(bt64);
    return -1;
  }
  for (int64_t i = 0; i < M; ++i)
    for (int64_t k = 0; k < K; ++k) a64[i * K + k] = oracle_decode(fmt, A[i * lda + k]);
  for (int64_t j = 0; j < N; ++j)
    for (int64_t k = 0; k < K; ++k)
      bt64[j * K + k] = (layout == ORACLE_NT) ? oracle_decode(fmt, B[j * ldb + k])
                                              : oracle_decode(fmt, B[k * ldb + j]);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t j = 0; j < N; ++j) {
      double d = 0.0, s = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double prod = a64[i * K + k] * bt64[j * K + k]; /* exact */
        d += prod;
        s += fabs(prod);
      }
      if (D) D[i * ldo + j] = d;
      if (S) S[i * ldo + j] = s;
    }
  }
  free(a64);
  free(bt64);
  return 0;
}

/* Selected elements (rows[t], cols[t]) for t < n: for spot checks at sizes
 * where the full product would take too long on the CPU. */
void oracle_gemm_entries(int layout, int fmt, int64_t K, const uint16_t* A, int64_t lda,
                         const uint16_t* B, int64_t ldb, int64_t n, const int64_t* rows,
                         const int64_t* cols, double* D, double* S) {
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < n; ++t) {
    dot_one(layout, fmt, K, A, lda, B, ldb, rows[t], cols[t], &D[t], &S[t]);
  }
}

/* Round every element of an array of doubles to the output format. */
void oracle_round_array(int fmt, int64_t n, const double* x, uint16_t* out) {
  for (int64_t t = 0; t < n; ++t) out[t] = oracle_round(fmt, x[t]);
}

/* Acceptance test over n elements.  d and s are the oracle's values, g the
 * device result as bit patterns of the output format.  Writes the number of
 * failing elements, the index and ratio |g - d| / tol of the worst element.
 * A non-finite g passes only where the correctly rounded d is the same
 * infinity. */
void oracle_check(int fmt, int64_t n, const double* d, const double* s, const uint16_t* g,
                  int64_t* n_fail, int64_t* worst_idx, double* worst_ratio) {
  int64_t fails = 0, widx = -1;
  double wr = 0.0;
  for (int64_t t = 0; t < n; ++t) {
    double gv = oracle_decode(fmt, g[t]);
    double tol = oracle_ulp(fmt, d[t]) + ldexp(s[t], -11);
    double ratio;
    if (!isfinite(gv)) {
      uint16_t want = oracle_round(fmt, d[t]);
      ratio = (isinf(gv) && want == g[t]) ? 0.0 : INFINITY;
    } else {
      ratio = fabs(gv - d[t]) / tol;
    }
    if (!(ratio <= 1.0)) ++fails;
    if (widx < 0 || ratio > wr) {
      wr = ratio;
      widx = t;
    }
  }
  *n_fail = fails;
  *worst_idx = widx;
  *worst_ratio = wr;
}

/* ---- FP8 block-scaled product --------------------------------------------
 *
 * CMU "TIRx" blog, section "Evaluation", "Kernel performance": FP8
 * block-scaled matrix multiplication, in which groups of input values share
 * scale factors.  The page fixes neither the FP8 encoding, nor the group
 * size, nor the scale format; TileFoundry's schedule tutorial, section 4,
 * lists fp8e4m3 operands as K-major on both sides.  The reading taken here
 * (the OCP microscaling layout): elements are E4M3 (1 sign, 4 exponent bits
 * with bias 7, 3 fraction bits; exponent field 0 is subnormal; S.1111.111 is
 * NaN; no infinities), and each group of 32 consecutive K values of a row
 * shares one E8M0 scale, the power of two 2^(e - 127) (e = 255 is NaN).
 * A is M x K (row i at A + i*lda), B is N x K (D = A @ B.T), the scales SA
 * are M x ceil(K/32) (row i at SA + i*ldsa), SB are N x ceil(K/32):
 *
 *   d[i][j] = sum_k dec8(A[i][k]) 2^(SA[i][k/32]-127) dec8(B[j][k]) 2^(SB[j][k/32]-127)
 *   s[i][j] = the same sum of absolute values
 *
 * Each scaled element is exact in double (4 significant bits, exponents
 * within +-136), so is every product; the sum runs in ascending k in
 * double.  The output format is BF16 (the same single rounding as above). */

double oracle_decode_e4m3(uint8_t v) {
  const int e = (v >> 3) & 15, m = v & 7;
  if (e == 15 && m == 7) return NAN;
  const double mag = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return (v & 0x80) ? -mag : mag;
}

double oracle_decode_e8m0(uint8_t e) { return e == 255 ? NAN : ldexp(1.0, (int)e - 127); }

static double mx_value(const uint8_t* X, int64_t ldx, const uint8_t* SX, int64_t ldsx, int64_t r,
                       int64_t k) {
  return oracle_decode_e4m3(X[r * ldx + k]) * oracle_decode_e8m0(SX[r * ldsx + k / 32]);
}

/* Full product (D, S: M x N with leading dimension ldo, either may be NULL).
 * Returns 0, or -1 if the scratch arrays cannot be allocated. */
int oracle_gemm_mx(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                   const uint8_t* SA, int64_t ldsa, const uint8_t* B, int64_t ldb,
                   const uint8_t* SB, int64_t ldsb, double* D, double* S, int64_t ldo) {
  double* a64 = (double*)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
  double* b64 = (double*)malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
  if (!a64 || !b64) {
    free(a64);
    free(b64);
    return -1;
  }
  for (int64_t i = 0; i < M; ++i)
    for (int64_t k = 0; k < K; ++k) a64[i * K + k] = mx_value(A, lda, SA, ldsa, i, k);
  for (int64_t j = 0; j < N; ++j)
    for (int64_t k = 0; k < K; ++k) b64[j * K + k] = mx_value(B, ldb, SB, ldsb, j, k);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t j = 0; j < N; ++j) {
      double d = 0.0, s = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double prod = a64[i * K + k] * b64[j * K + k]; /* exact */
        d += prod;
        s += fabs(prod);
      }
      if (D) D[i * ldo + j] = d;
      if (S) S[i * ldo + j] = s;
    }
  }
  free(a64);
  free(b64);
  return 0;
}

/* Selected elements (rows[t], cols[t]) for t < n. */
void oracle_gemm_mx_entries(int64_t K, const uint8_t* A, int64_t lda, const uint8_t* SA,
                            int64_t ldsa, const uint8_t* B, int64_t ldb, const uint8_t* SB,
                            int64_t ldsb, int64_t n, const int64_t* rows, const int64_t* cols,
                            double* D, double* S) {
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < n; ++t) {
    double d = 0.0, s = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double prod = mx_value(A, lda, SA, ldsa, rows[t], k) * mx_value(B, ldb, SB, ldsb, cols[t], k);
      d += prod;
      s += fabs(prod);
    }
    D[t] = d;
    S[t] = s;
  }
}
