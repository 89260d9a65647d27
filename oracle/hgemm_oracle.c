/*
 * hgemm_oracle.c -- plain, slow, obviously-correct CPU oracle for dense
 * half-precision GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this code.  The HIP library shares
 * no code, header, table or helper with it.
 *
 * What it computes (the definition, written out):
 *
 *   ref[m][n] = RNE_dtype( sum_{k=0..K-1} double(A[m][k]) * double(Bop[k][n]) )
 *
 *   - The naive triple loop of "tcgen05 for dummies" (Chinese translation,
 *     "[译] tcgen05 入门：从零实现 B200 GEMM"), section "Recap: how to write a
 *     high-performance matmul kernel" (the `matmul` listing): one dot product
 *     per output element, accumulator initialised to zero, summed along K.
 *   - Layouts from the kernel header comment of "HGEMM: WMMA 与 MMA PTX 代码学习"
 *     (full listing section): NN = A, B, C all row-major; TN = A row-major
 *     MxK, B stored "column-major", i.e. as an N x K row-major array Bt, so
 *     Bop[k][n] = Bt[n][k].
 *   - Half-precision inputs, wide accumulation, then one conversion of the
 *     sum back to the half type: section 3 of "MTT S4000 张量核心 GEMM 优化…"
 *     (steps 4 and 7 of its outline).  The oracle accumulates in FP64 (every
 *     f16*f16 and bf16*bf16 product is exact in FP64) in ascending k and
 *     rounds the FP64 sum directly to the output type.
 *   - Rounding is IEEE-754 round-to-nearest, ties-to-even, with gradual
 *     underflow and overflow to +-infinity, implemented below from the format
 *     definitions (binary16: 1/5/10 bits, bias 15; bfloat16: 1/8/7 bits,
 *     bias 127).  The pages convert with round-to-nearest intrinsics in the
 *     tcgen05 translation's epilogue and the S4000 post's final store.
 *
 * Blocking, fusion or reordering: none.  OpenMP only splits the m loop
 * across threads; every element is computed by the same sequential k loop.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared (no -ffast-math).
 * A build with -DORACLE_MUTATION=<n> plants one deliberate mistake; the test
 * suite uses those builds to show that its pins catch each mistake.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTATION
#define ORACLE_MUTATION 0
#endif

enum { ORACLE_F16 = 0, ORACLE_BF16 = 1 };
enum { ORACLE_TN = 0, ORACLE_NN = 1 };

/* ---------------------------------------------------------------------- */
/* Format parameters.                                                      */
/*   p     = significand precision in bits, implicit bit included          */
/*   emin  = exponent of the smallest normal number                        */
/*   emax  = exponent of the largest finite number                         */
/*   ebits = width of the biased exponent field                            */
/* ---------------------------------------------------------------------- */
typedef struct {
  int p, emin, emax, ebits, bias;
} fmt_t;

static const fmt_t FMT_F16 = {11, -14, 15, 5, 15};
#if ORACLE_MUTATION == 5
/* planted mistake: wrong bfloat16 exponent bias */
static const fmt_t FMT_BF16 = {8, -126, 127, 8, 126};
#else
static const fmt_t FMT_BF16 = {8, -126, 127, 8, 127};
#endif

static const fmt_t *fmt_of(int dtype) {
  return dtype == ORACLE_BF16 ? &FMT_BF16 : &FMT_F16;
}

/* Decode a 16-bit pattern to its exact value.  */
static double decode16(uint16_t bits, const fmt_t *f) {
  const int fbits = f->p - 1;
  const int sign = bits >> 15;
  const int e = (bits >> fbits) & ((1 << f->ebits) - 1);
  const int frac = bits & ((1 << fbits) - 1);
  double v;
  if (e == 0) {
    /* subnormal (or zero): frac * 2^(emin - fbits) */
    v = ldexp((double)frac, f->emin - fbits);
  } else if (e == (1 << f->ebits) - 1) {
    v = frac ? NAN : INFINITY;
  } else {
    /* normal: (2^fbits + frac) * 2^(e - bias - fbits) */
    v = ldexp((double)((1 << fbits) + frac), e - f->bias - fbits);
  }
  return sign ? -v : v;
}

/* Round a double to the nearest value of the format, ties to even.
 * Returns the rounded value as a double (possibly +-inf).            */
static double round_to_format(double x, const fmt_t *f) {
  if (isnan(x) || isinf(x) || x == 0.0) return x;
  const double ax = fabs(x);
  /* exponent of ax: ax = m * 2^e with 1 <= m < 2 */
  int e2;
  frexp(ax, &e2); /* ax = fr * 2^e2, 0.5 <= fr < 1 */
  int e = e2 - 1;
  if (e < f->emin) e = f->emin; /* subnormal range shares emin's quantum */
  const int qexp = e - (f->p - 1); /* quantum (unit in the last place) */
  const double r = ldexp(ax, -qexp); /* exact: scaling by a power of two */
  const double fl = floor(r);
  const double d = r - fl; /* exact: r has at most 53 significant bits */
  double n;
#if ORACLE_MUTATION == 3
  /* planted mistake: ties rounded away from zero */
  n = (d >= 0.5) ? fl + 1.0 : fl;
#elif ORACLE_MUTATION == 4
  /* planted mistake: truncation instead of rounding */
  n = fl;
  (void)d;
#else
  if (d > 0.5) {
    n = fl + 1.0;
  } else if (d < 0.5) {
    n = fl;
  } else {
    n = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0; /* tie: pick the even one */
  }
#endif
  double v = ldexp(n, qexp);
  /* overflow: anything that rounds beyond the largest finite value */
  const double maxfinite =
      ldexp((double)((1 << f->p) - 1), f->emax - (f->p - 1));
  if (v > maxfinite) v = INFINITY;
  return x < 0 ? -v : v;
}

/* Encode a value that is exactly representable in the format (or +-inf,
 * or NaN) as its 16-bit pattern.                                      */
static uint16_t encode16(double v, const fmt_t *f) {
  const int fbits = f->p - 1;
  const int emask = (1 << f->ebits) - 1;
  if (isnan(v)) return (uint16_t)((emask << fbits) | (1 << (fbits - 1)));
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double av = fabs(v);
  if (isinf(av)) return (uint16_t)(sign | (emask << fbits));
  if (av == 0.0) return sign;
  int e2;
  frexp(av, &e2);
  int e = e2 - 1;
  if (e < f->emin) {
    /* subnormal: av = frac * 2^(emin - fbits) */
    double frac = ldexp(av, -(f->emin - fbits));
    return (uint16_t)(sign | (uint16_t)frac);
  }
  double sig = ldexp(av, -(e - fbits)); /* in [2^fbits, 2^(fbits+1)) */
  int frac = (int)sig - (1 << fbits);
  return (uint16_t)(sign | ((e + f->bias) << fbits) | frac);
}

/* ---------------------------------------------------------------------- */
/* Exported array helpers (checked exhaustively by the oracle's own pins). */
/* ---------------------------------------------------------------------- */
void oracle_decode_array(int dtype, const uint16_t *in, double *out,
                         int64_t n) {
  const fmt_t *f = fmt_of(dtype);
  for (int64_t i = 0; i < n; ++i) out[i] = decode16(in[i], f);
}

void oracle_round_array(int dtype, const double *in, uint16_t *out,
                        int64_t n) {
  const fmt_t *f = fmt_of(dtype);
  for (int64_t i = 0; i < n; ++i) out[i] = encode16(round_to_format(in[i], f), f);
}

/* ---------------------------------------------------------------------- */
/* GEMM.                                                                   */
/* ---------------------------------------------------------------------- */

/* Bop[k][n] for the given layout. */
static inline uint16_t bop(int layout, const uint16_t *B, int64_t N, int64_t K,
                           int64_t k, int64_t n) {
#if ORACLE_MUTATION == 2
  /* planted mistake: both layouts read B as if it were stored N x K */
  (void)layout;
  (void)N;
  return B[n * K + k];
#else
  return layout == ORACLE_TN ? B[n * K + k] : B[k * N + n];
#endif
}

/* One output element, the definition written out. */
static double dot(int layout, const double *lut, const uint16_t *A,
                  const uint16_t *B, int64_t N, int64_t K, int64_t m,
                  int64_t n) {
  double acc = 0.0;
#if ORACLE_MUTATION == 1
  /* planted mistake: the last k term is dropped */
  const int64_t kend = K > 0 ? K - 1 : 0;
#else
  const int64_t kend = K;
#endif
  for (int64_t k = 0; k < kend; ++k) {
    const double a = lut[A[m * K + k]];
    const double b = lut[bop(layout, B, N, K, k, n)];
#if ORACLE_MUTATION == 6
    /* planted mistake: wrong sign on odd k */
    acc += (k & 1) ? -a * b : a * b;
#else
    acc += a * b;
#endif
  }
  return acc;
}

static double *make_lut(int dtype) {
  const fmt_t *f = fmt_of(dtype);
  double *lut = (double *)malloc(sizeof(double) * 65536);
  if (!lut) return NULL;
  for (int i = 0; i < 65536; ++i) lut[i] = decode16((uint16_t)i, f);
  return lut;
}

static int check_args(int layout, int dtype, int64_t M, int64_t N, int64_t K) {
  if (layout != ORACLE_TN && layout != ORACLE_NN) return -1;
  if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
  if (M < 0 || N < 0 || K < 0) return -1;
  return 0;
}

/* Full output for rows [row_begin, row_end) of C (C points at row 0).
 * Returns 0 on success, -1 on bad arguments, -2 on allocation failure. */
int oracle_hgemm_rows(int layout, int dtype, int64_t M, int64_t N, int64_t K,
                      const uint16_t *A, const uint16_t *B, uint16_t *C,
                      int64_t row_begin, int64_t row_end) {
  if (check_args(layout, dtype, M, N, K)) return -1;
  if (row_begin < 0 || row_end > M || row_begin > row_end) return -1;
  double *lut = make_lut(dtype);
  if (!lut) return -2;
  const fmt_t *f = fmt_of(dtype);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = row_begin; m < row_end; ++m) {
    for (int64_t n = 0; n < N; ++n) {
      const double s = dot(layout, lut, A, B, N, K, m, n);
      C[m * N + n] = encode16(round_to_format(s, f), f);
    }
  }
  free(lut);
  return 0;
}

int oracle_hgemm(int layout, int dtype, int64_t M, int64_t N, int64_t K,
                 const uint16_t *A, const uint16_t *B, uint16_t *C) {
  return oracle_hgemm_rows(layout, dtype, M, N, K, A, B, C, 0, M);
}

/* Selected output elements: out[i] = ref[rows[i]][cols[i]]. */
int oracle_hgemm_sampled(int layout, int dtype, int64_t M, int64_t N,
                         int64_t K, const uint16_t *A, const uint16_t *B,
                         const int64_t *rows, const int64_t *cols,
                         int64_t count, uint16_t *out) {
  if (check_args(layout, dtype, M, N, K)) return -1;
  for (int64_t i = 0; i < count; ++i)
    if (rows[i] < 0 || rows[i] >= M || cols[i] < 0 || cols[i] >= N) return -1;
  double *lut = make_lut(dtype);
  if (!lut) return -2;
  const fmt_t *f = fmt_of(dtype);
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t i = 0; i < count; ++i) {
#if ORACLE_MUTATION == 12
    /* planted mistake: row and column of the sample swapped */
    const double s = dot(layout, lut, A, B, N, K, cols[i], rows[i]);
#else
    const double s = dot(layout, lut, A, B, N, K, rows[i], cols[i]);
#endif
    out[i] = encode16(round_to_format(s, f), f);
  }
  free(lut);
  return 0;
}

/* ---------------------------------------------------------------------- */
/* General form: operation flags, leading dimensions, alpha and beta.      */
/*                                                                         */
/*   C[m][n] = RNE( alpha * S[m][n] + beta * Cin[m][n] ),                  */
/*   S[m][n] = sum_{k<K} opA(A)[m][k] * opB(B)[k][n]   (FP64, ascending k)  */
/*                                                                         */
/* Row-major storage throughout:                                           */
/*   opA 0: A is M x K,        opA(A)[m][k] = A[m*lda + k]                  */
/*   opA 1: A is stored K x M, opA(A)[m][k] = A[k*lda + m]                  */
/*   opB 0: B is K x N,        opB(B)[k][n] = B[k*ldb + n]                  */
/*   opB 1: B is stored N x K, opB(B)[k][n] = B[n*ldb + k]                  */
/*   C and Cin are M x N with leading dimensions ldc and ldcin.            */
/* The pages' two layouts are (opA, opB) = (0, 1) for TN and (0, 0) for    */
/* NN with packed leading dimensions, alpha = 1 and beta = 0.  The pages   */
/* stop at C = A*B; the alpha/beta update is the usual BLAS gemm one,      */
/* beta == 0 meaning Cin is not read at all (it may hold NaN).             */
/* ---------------------------------------------------------------------- */
static inline uint16_t gen_a(int opA, const uint16_t *A, int64_t lda,
                             int64_t m, int64_t k) {
#if ORACLE_MUTATION == 8
  /* planted mistake: a transposed A read as if it were not */
  (void)opA;
  return A[m * lda + k];
#else
  return opA ? A[k * lda + m] : A[m * lda + k];
#endif
}

static inline uint16_t gen_b(int opB, const uint16_t *B, int64_t ldb, int64_t N,
                             int64_t K, int64_t k, int64_t n) {
#if ORACLE_MUTATION == 9
  /* planted mistake: the leading dimension of B ignored (packed stride) */
  (void)ldb;
  return opB ? B[n * K + k] : B[k * N + n];
#else
  (void)N;
  (void)K;
  return opB ? B[n * ldb + k] : B[k * ldb + n];
#endif
}

static double gen_element(int opA, int opB, const double *lut, int64_t N,
                          int64_t K, double alpha, const uint16_t *A,
                          int64_t lda, const uint16_t *B, int64_t ldb,
                          double beta, const uint16_t *Cin, int64_t ldcin,
                          int64_t m, int64_t n) {
  double acc = 0.0;
  for (int64_t k = 0; k < K; ++k)
    acc += lut[gen_a(opA, A, lda, m, k)] * lut[gen_b(opB, B, ldb, N, K, k, n)];
  double v = alpha * acc;
#if ORACLE_MUTATION == 7
  /* planted mistake: beta ignored */
  (void)beta;
  (void)Cin;
  (void)ldcin;
#else
  if (beta != 0.0) v += beta * lut[Cin[m * ldcin + n]];
#endif
  return v;
}

static int check_gen(int opA, int opB, int dtype, int64_t M, int64_t N,
                     int64_t K, int64_t lda, int64_t ldb, int64_t ldcin,
                     double beta, const uint16_t *Cin) {
  if ((opA != 0 && opA != 1) || (opB != 0 && opB != 1)) return -1;
  if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
  if (M < 0 || N < 0 || K < 0) return -1;
  if (lda < (opA ? M : K) || ldb < (opB ? K : N)) return -1;
  if (beta != 0.0 && (Cin == NULL || ldcin < N)) return -1;
  return 0;
}

/* Rows [row_begin, row_end) of the general form; C[m*ldc + n]. */
int oracle_gemm_rows(int opA, int opB, int dtype, int64_t M, int64_t N,
                     int64_t K, double alpha, const uint16_t *A, int64_t lda,
                     const uint16_t *B, int64_t ldb, double beta,
                     const uint16_t *Cin, int64_t ldcin, uint16_t *C,
                     int64_t ldc, int64_t row_begin, int64_t row_end) {
  if (check_gen(opA, opB, dtype, M, N, K, lda, ldb, ldcin, beta, Cin)) return -1;
  if (ldc < N || row_begin < 0 || row_end > M || row_begin > row_end) return -1;
  double *lut = make_lut(dtype);
  if (!lut) return -2;
  const fmt_t *f = fmt_of(dtype);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = row_begin; m < row_end; ++m)
    for (int64_t n = 0; n < N; ++n) {
      const double v = gen_element(opA, opB, lut, N, K, alpha, A, lda, B, ldb,
                                   beta, Cin, ldcin, m, n);
      C[m * ldc + n] = encode16(round_to_format(v, f), f);
    }
  free(lut);
  return 0;
}

/* Selected elements of the general form: out[i] = C[rows[i]][cols[i]]. */
int oracle_gemm_sampled(int opA, int opB, int dtype, int64_t M, int64_t N,
                        int64_t K, double alpha, const uint16_t *A,
                        int64_t lda, const uint16_t *B, int64_t ldb,
                        double beta, const uint16_t *Cin, int64_t ldcin,
                        const int64_t *rows, const int64_t *cols,
                        int64_t count, uint16_t *out) {
  if (check_gen(opA, opB, dtype, M, N, K, lda, ldb, ldcin, beta, Cin)) return -1;
  for (int64_t i = 0; i < count; ++i)
    if (rows[i] < 0 || rows[i] >= M || cols[i] < 0 || cols[i] >= N) return -1;
  double *lut = make_lut(dtype);
  if (!lut) return -2;
  const fmt_t *f = fmt_of(dtype);
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t i = 0; i < count; ++i) {
#if ORACLE_MUTATION == 10
    /* planted mistake: row and column of the sample swapped */
    const double v = gen_element(opA, opB, lut, N, K, alpha, A, lda, B, ldb,
                                 beta, Cin, ldcin, cols[i], rows[i]);
#elif ORACLE_MUTATION == 11
    /* planted mistake: the old C read with the packed stride N, not ldcin */
    const double v = gen_element(opA, opB, lut, N, K, alpha, A, lda, B, ldb,
                                 beta, Cin, N, rows[i], cols[i]);
#else
    const double v = gen_element(opA, opB, lut, N, K, alpha, A, lda, B, ldb,
                                 beta, Cin, ldcin, rows[i], cols[i]);
#endif
    out[i] = encode16(round_to_format(v, f), f);
  }
  free(lut);
  return 0;
}

int oracle_mutation(void) { return ORACLE_MUTATION; }
