/*
 * Reference SGEMM oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * may load this library.  The product path (the HIP library and its Python
 * binding) never calls it and shares no code with it.
 *
 * What it computes is the plain definition of the operation from the page
 * "GEMM 优化之路" (section on the problem statement and performance limit):
 * C = alpha * A * B + beta * C, with A of size M x K, B of size K x N and C of
 * size M x N, all row-major FP32.  Leading dimensions are explicit here
 * (A(i,k) = A[i*lda + k], B(k,j) = B[k*ldb + j], C(i,j) = C[i*ldc + j]); the
 * page uses the minimal ones (K, N, N).
 *
 * Transposed operands (the A^T*B and A*B^T cases of the gsyq.cn guide,
 * section 6.4 step 8): with transa set, the stored matrix is K x M and
 * A(i,k) = A[k*lda + i]; with transb set, the stored matrix is N x K and
 * B(k,j) = B[j*ldb + k].  Only the indexing changes; the sums are the same.
 *
 * Arithmetic is FP64 throughout:
 *   s_ij = sum over k = 0 .. K-1, ascending, of (double)A(i,k) * (double)B(k,j)
 *          with one accumulator per output element;
 *   t_ij = sum over the same k of |(double)A(i,k) * (double)B(k,j)|;
 *   r_ij = (double)alpha * s_ij            if beta == 0 (C is not read),
 *          (double)alpha * s_ij + (double)beta * (double)C(i,j)   otherwise.
 * The product of two FP32 numbers is exact in FP64 (24 + 24 <= 53 bits), so
 * only the additions round.  r_ij is returned unrounded; the caller rounds it
 * to FP32 when it needs the FP32 result.
 *
 * Low-precision inputs (oracle_gemm_lowp): the mixed-precision product of
 * the gsyq.cn guide, section 5.1 (matrix units take 16-bit A and B and
 * accumulate into FP32), with A and B stored as 16-bit patterns in one of two
 * formats, decoded exactly from their definitions:
 *   - bfloat16: the upper 16 bits of an IEEE binary32 number;
 *   - IEEE binary16: 1 sign bit, 5 exponent bits with bias 15, 10 fraction
 *     bits; exponent 0 holds subnormals (fraction * 2^-24), exponent 31
 *     infinities and NaNs.
 * C, alpha and beta stay FP32 and the sums are the FP64 sums above: the
 * product of two 16-bit values is exact in FP64 as well.
 * The same with 8-bit A and B (oracle_gemm_fp8), in the two OCP 8-bit
 * floating-point formats:
 *   - E4M3: 1 sign, 4 exponent bits with bias 7, 3 fraction bits; exponent 0
 *     holds subnormals (fraction * 2^-9); the pattern with all exponent and
 *     fraction bits set is NaN; there are no infinities;
 *   - E5M2: 1 sign, 5 exponent bits with bias 15, 2 fraction bits; exponent 0
 *     holds subnormals (fraction * 2^-16), exponent 31 infinities and NaNs.
 *
 * The loop nest follows the CPU reference on the same page (its complete
 * listing): rows outer, then k, then columns, with a row of accumulators.
 * Threads split the rows; nothing else is blocked, fused or reordered.
 * Build with plain -O2 and no -ffast-math so the compiler may not reassociate
 * the per-element sums.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int M, N, K;
  int ta, tb;  /* transposed storage of A / B */
  double alpha, beta;
  const float *A, *B, *C;
  /* 16-bit or 8-bit storage of A and B (dt != DT_F32): bit patterns, same
   * indexing */
  int dt;
  const uint16_t *A16, *B16;
  const uint8_t *A8, *B8;
  long lda, ldb, ldc;
  double *R, *T;
  long ldr, ldt;
  /* point mode */
  int npts;
  const int *rows, *cols;
  /* work split */
  int first, last;
} job_t;

/* Element formats. */
enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2, DT_E4M3 = 3, DT_E5M2 = 4 };

/* bfloat16: the pattern is the upper half of an IEEE binary32 number. */
static double bf16_value(uint16_t h) {
  const uint32_t w = (uint32_t)h << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

/* IEEE binary16: (-1)^s * 2^(e-15) * (1 + m/1024) for 0 < e < 31,
 * (-1)^s * 2^-14 * (m/1024) for e == 0, infinity or NaN for e == 31. */
static double f16_value(uint16_t h) {
  const int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

static double value16(int dt, uint16_t h) {
  return dt == DT_BF16 ? bf16_value(h) : f16_value(h);
}

/* E4M3: (-1)^s * 2^(e-7) * (1 + m/8) for e > 0, (-1)^s * 2^-6 * (m/8) for
 * e == 0; exponent and fraction all ones is NaN. */
static double e4m3_value(uint8_t b) {
  const int s = (b >> 7) & 1, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp((double)(8 + m), e - 10);
  return s != 0 ? -v : v;
}

/* E5M2: (-1)^s * 2^(e-15) * (1 + m/4) for 0 < e < 31, (-1)^s * 2^-14 * (m/4)
 * for e == 0, infinity or NaN for e == 31. */
static double e5m2_value(uint8_t b) {
  const int s = (b >> 7) & 1, e = (b >> 2) & 31, m = b & 3;
  double v;
  if (e == 31)
    v = m ? NAN : INFINITY;
  else if (e == 0)
    v = ldexp((double)m, -16);
  else
    v = ldexp((double)(4 + m), e - 17);
  return (s != 0) ? -v : v;
}

static double value8(int dt, uint8_t b) {
  return dt == DT_E4M3 ? e4m3_value(b) : e5m2_value(b);
}

/* Element (i,k) of A and (k,j) of B under the storage flags. */
static double a_at(const job_t *j, int i, int k) {
  if (j->dt >= DT_E4M3)
    return value8(j->dt, j->ta ? j->A8[(long)k * j->lda + i]
                               : j->A8[(long)i * j->lda + k]);
  if (j->dt != DT_F32)
    return value16(j->dt, j->ta ? j->A16[(long)k * j->lda + i]
                                : j->A16[(long)i * j->lda + k]);
  return (double)(j->ta ? j->A[(long)k * j->lda + i] : j->A[(long)i * j->lda + k]);
}
static double b_at(const job_t *j, int k, int c) {
  if (j->dt >= DT_E4M3)
    return value8(j->dt, j->tb ? j->B8[(long)c * j->ldb + k]
                               : j->B8[(long)k * j->ldb + c]);
  if (j->dt != DT_F32)
    return value16(j->dt, j->tb ? j->B16[(long)c * j->ldb + k]
                                : j->B16[(long)k * j->ldb + c]);
  return (double)(j->tb ? j->B[(long)c * j->ldb + k] : j->B[(long)k * j->ldb + c]);
}

/* Rows [first, last) of the full product. */
static void *full_rows(void *arg) {
  job_t *j = (job_t *)arg;
  for (int i = j->first; i < j->last; ++i) {
    double *r = j->R + (long)i * j->ldr;
    double *t = j->T ? j->T + (long)i * j->ldt : NULL;
    for (int c = 0; c < j->N; ++c) r[c] = 0.0;
    if (t)
      for (int c = 0; c < j->N; ++c) t[c] = 0.0;
    for (int k = 0; k < j->K; ++k) {
      const double a = a_at(j, i, k);
      for (int c = 0; c < j->N; ++c) {
        const double p = a * b_at(j, k, c);
        r[c] += p;
        if (t) t[c] += fabs(p);
      }
    }
    for (int c = 0; c < j->N; ++c) {
      double v = j->alpha * r[c];
      if (j->beta != 0.0) v += j->beta * (double)j->C[(long)i * j->ldc + c];
      r[c] = v;
    }
  }
  return NULL;
}

/* Points [first, last) of the point list: one dot product each. */
static void *points(void *arg) {
  job_t *j = (job_t *)arg;
  for (int p = j->first; p < j->last; ++p) {
    const int i = j->rows[p], c = j->cols[p];
    double s = 0.0, a = 0.0;
    for (int k = 0; k < j->K; ++k) {
      const double q = a_at(j, i, k) * b_at(j, k, c);
      s += q;
      a += fabs(q);
    }
    double v = j->alpha * s;
    if (j->beta != 0.0) v += j->beta * (double)j->C[(long)i * j->ldc + c];
    j->R[p] = v;
    if (j->T) j->T[p] = a;
  }
  return NULL;
}

static int check_args(int ta, int tb, int M, int N, int K, int lda, int ldb,
                      int ldc) {
  if (M < 0 || N < 0 || K < 0) return -1;
  const int a_cols = ta ? M : K, b_cols = tb ? K : N;
  if (lda < (a_cols > 1 ? a_cols : 1)) return -2;
  if (ldb < (b_cols > 1 ? b_cols : 1)) return -2;
  if (ldc < (N > 1 ? N : 1)) return -2;
  return 0;
}

static void run_split(void *(*fn)(void *), job_t *proto, int count,
                      int nthreads) {
  if (count <= 0) return;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > count) nthreads = count;
  if (nthreads > 256) nthreads = 256;
  pthread_t tid[256];
  job_t jobs[256];
  int started[256];
  for (int w = 0; w < nthreads; ++w) {
    jobs[w] = *proto;
    jobs[w].first = (int)((long)count * w / nthreads);
    jobs[w].last = (int)((long)count * (w + 1) / nthreads);
    started[w] = (w > 0) && pthread_create(&tid[w], NULL, fn, &jobs[w]) == 0;
    if (w > 0 && !started[w]) fn(&jobs[w]); /* no thread: run inline */
  }
  fn(&jobs[0]);
  for (int w = 1; w < nthreads; ++w)
    if (started[w]) pthread_join(tid[w], NULL);
}

/*
 * Full product.  R receives r_ij (ldr >= N), T receives t_ij (ldt >= N) or is
 * NULL to skip the magnitude sum (the timing mode).  ta / tb select the
 * transposed storage of A / B.  Returns 0, or -1 for a negative size, -2 for
 * a leading dimension that is too small.
 */
int oracle_sgemm_ex(int ta, int tb, int M, int N, int K, float alpha,
                    const float *A, int lda, const float *B, int ldb,
                    float beta, const float *C, int ldc, double *R, int ldr,
                    double *T, int ldt, int nthreads) {
  int e = check_args(ta, tb, M, N, K, lda, ldb, ldc);
  if (e) return e;
  if (ldr < N || (T && ldt < N)) return -2;
  job_t j;
  memset(&j, 0, sizeof j);
  j.M = M; j.N = N; j.K = K;
  j.ta = ta != 0; j.tb = tb != 0;
  j.alpha = (double)alpha; j.beta = (double)beta;
  j.A = A; j.B = B; j.C = C;
  j.lda = lda; j.ldb = ldb; j.ldc = ldc;
  j.R = R; j.T = T; j.ldr = ldr; j.ldt = ldt;
  if (N > 0) run_split(full_rows, &j, M, nthreads);
  return 0;
}

int oracle_sgemm(int M, int N, int K, float alpha, const float *A, int lda,
                 const float *B, int ldb, float beta, const float *C, int ldc,
                 double *R, int ldr, double *T, int ldt, int nthreads) {
  return oracle_sgemm_ex(0, 0, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                         R, ldr, T, ldt, nthreads);
}

/*
 * Selected outputs (rows[p], cols[p]) for p < npts, each an independent dot
 * product with the same definition as above; r_out[p] = r_ij, t_out[p] = t_ij
 * (t_out may be NULL).  Used where the full product would take too long.
 * Returns 0, -1/-2 as above, or -3 for a point outside the M x N window.
 */
int oracle_sgemm_points_ex(int ta, int tb, int M, int N, int K, float alpha,
                           const float *A, int lda, const float *B, int ldb,
                           float beta, const float *C, int ldc, int npts,
                           const int *rows, const int *cols, double *r_out,
                           double *t_out, int nthreads) {
  int e = check_args(ta, tb, M, N, K, lda, ldb, ldc);
  if (e) return e;
  for (int p = 0; p < npts; ++p)
    if (rows[p] < 0 || rows[p] >= M || cols[p] < 0 || cols[p] >= N) return -3;
  job_t j;
  memset(&j, 0, sizeof j);
  j.M = M; j.N = N; j.K = K;
  j.alpha = (double)alpha; j.beta = (double)beta;
  j.A = A; j.B = B; j.C = C;
  j.lda = lda; j.ldb = ldb; j.ldc = ldc;
  j.ta = ta != 0; j.tb = tb != 0;
  j.R = r_out; j.T = t_out;
  j.npts = npts; j.rows = rows; j.cols = cols;
  run_split(points, &j, npts, nthreads);
  return 0;
}

int oracle_sgemm_points(int M, int N, int K, float alpha, const float *A,
                        int lda, const float *B, int ldb, float beta,
                        const float *C, int ldc, int npts, const int *rows,
                        const int *cols, double *r_out, double *t_out,
                        int nthreads) {
  return oracle_sgemm_points_ex(0, 0, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                ldc, npts, rows, cols, r_out, t_out, nthreads);
}

/*
 * The same products with A and B in a 16-bit format: dt = 1 for bfloat16,
 * 2 for IEEE binary16 (bit patterns as stored).  C, alpha, beta, R and T as
 * in oracle_sgemm_ex.  Returns 0, -1/-2 as there, or -4 for an unknown dt.
 */
int oracle_gemm_lowp(int dt, int ta, int tb, int M, int N, int K, float alpha,
                     const uint16_t *A, int lda, const uint16_t *B, int ldb,
                     float beta, const float *C, int ldc, double *R, int ldr,
                     double *T, int ldt, int nthreads) {
  if (dt != DT_BF16 && dt != DT_F16) return -4;
  int e = check_args(ta, tb, M, N, K, lda, ldb, ldc);
  if (e) return e;
  if (ldr < N || (T && ldt < N)) return -2;
  job_t j;
  memset(&j, 0, sizeof j);
  j.M = M; j.N = N; j.K = K;
  j.ta = ta != 0; j.tb = tb != 0;
  j.alpha = (double)alpha; j.beta = (double)beta;
  j.dt = dt; j.A16 = A; j.B16 = B; j.C = C;
  j.lda = lda; j.ldb = ldb; j.ldc = ldc;
  j.R = R; j.T = T; j.ldr = ldr; j.ldt = ldt;
  if (N > 0) run_split(full_rows, &j, M, nthreads);
  return 0;
}

/* Selected outputs of the 16-bit product, as oracle_sgemm_points_ex. */
int oracle_gemm_lowp_points(int dt, int ta, int tb, int M, int N, int K,
                            float alpha, const uint16_t *A, int lda,
                            const uint16_t *B, int ldb, float beta,
                            const float *C, int ldc, int npts, const int *rows,
                            const int *cols, double *r_out, double *t_out,
                            int nthreads) {
  if (dt != DT_BF16 && dt != DT_F16) return -4;
  int e = check_args(ta, tb, M, N, K, lda, ldb, ldc);
  if (e) return e;
  for (int p = 0; p < npts; ++p)
    if (rows[p] < 0 || rows[p] >= M || cols[p] < 0 || cols[p] >= N) return -3;
  job_t j;
  memset(&j, 0, sizeof j);
  j.M = M; j.N = N; j.K = K;
  j.ta = ta != 0; j.tb = tb != 0;
  j.alpha = (double)alpha; j.beta = (double)beta;
  j.dt = dt; j.A16 = A; j.B16 = B; j.C = C;
  j.lda = lda; j.ldb = ldb; j.ldc = ldc;
  j.npts = npts; j.rows = rows; j.cols = cols;
  j.R = r_out; j.T = t_out;
  run_split(points, &j, npts, nthreads);
  return 0;
}

/*
 * The same products with A and B in an 8-bit format: dt = 3 for E4M3, 4 for
 * E5M2 (bit patterns as stored).  C, alpha, beta, R and T as in
 * oracle_sgemm_ex.  Returns 0, -1/-2 as there, or -4 for an unknown dt.
 */
int oracle_gemm_fp8(int dt, int ta, int tb, int M, int N, int K, float alpha,
                    const uint8_t *A, int lda, const uint8_t *B, int ldb,
                    float beta, const float *C, int ldc, double *R, int ldr,
                    double *T, int ldt, int nthreads) {
  if (dt != DT_E4M3 && dt != DT_E5M2) return -4;
  int e = check_args(ta, tb, M, N, K, lda, ldb, ldc);
  if (e) return e;
  if (ldr < N || (T && ldt < N)) return -2;
  job_t j;
  memset(&j, 0, sizeof j);
  j.M = M; j.N = N; j.K = K;
  j.ta = ta != 0; j.tb = tb != 0;
  j.alpha = (double)alpha; j.beta = (double)beta;
  j.dt = dt; j.A8 = A; j.B8 = B; j.C = C;
  j.lda = lda; j.ldb = ldb; j.ldc = ldc;
  j.R = R; j.T = T; j.ldr = ldr; j.ldt = ldt;
  if (N > 0) run_split(full_rows, &j, M, nthreads);
  return 0;
}

/* Selected outputs of the 8-bit product, as oracle_sgemm_points_ex. */
int oracle_gemm_fp8_points(int dt, int ta, int tb, int M, int N, int K,
                           float alpha, const uint8_t *A, int lda,
                           const uint8_t *B, int ldb, float beta,
                           const float *C, int ldc, int npts, const int *rows,
                           const int *cols, double *r_out, double *t_out,
                           int nthreads) {
  if (dt != DT_E4M3 && dt != DT_E5M2) return -4;
  int e = check_args(ta, tb, M, N, K, lda, ldb, ldc);
  if (e) return e;
  for (int p = 0; p < npts; ++p)
    if (rows[p] < 0 || rows[p] >= M || cols[p] < 0 || cols[p] >= N) return -3;
  job_t j;
  memset(&j, 0, sizeof j);
  j.M = M; j.N = N; j.K = K;
  j.ta = ta != 0; j.tb = tb != 0;
  j.alpha = (double)alpha; j.beta = (double)beta;
  j.dt = dt; j.A8 = A; j.B8 = B; j.C = C;
  j.lda = lda; j.ldb = ldb; j.ldc = ldc;
  j.rows = rows; j.cols = cols; j.npts = npts;
  j.R = r_out; j.T = t_out;
  run_split(points, &j, npts, nthreads);
  return 0;
}
