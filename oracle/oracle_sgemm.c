/*
 * oracle_sgemm.c -- CPU oracle for single-precision GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no source, header, constant
 * or build step with the HIP library; it re-states the problem from the pages.
 *
 * What it computes (all four pages state the same problem; the kernels in
 * "Shared Memory Tiling" (the kernel listing and its epilogue line),
 * "Vectorized Memory Access: 128-bit Loads and Stores" (section "The Kernel")
 * and "Warp Tiling: A Third Level of Tiling" (section "The Kernel") all end in
 * the update alpha * (sum over k of A[i][k]*B[k][j]) + beta * C[i][j]):
 *
 *     C_out[i,j] = round_to_fp32( alpha * sum_{k=0}^{K-1} A[i,k] * B[k,j]
 *                                 + beta * C_in[i,j] )
 *
 * for 0 <= i < M, 0 <= j < N, with row-major operands addressed through
 * leading dimensions: X[r,c] = X_ptr[r*ldX + c].  The pages use the tight
 * strides K, N and N; leading dimensions generalise that without changing the
 * arithmetic.  No other element of C's allocation is read or written.
 *
 * Precision: every product of two fp32 values is exact in fp64 (24+24 bits of
 * significand fit in 53), the sum runs in fp64 in ascending k order, the
 * epilogue is evaluated in fp64 and rounded once to fp32 (round to nearest
 * even, the C default).  Build without -ffast-math.
 *
 * Loop order: rows are independent (one OpenMP task per row i, so results do
 * not depend on the thread count).  Within a row the loop is i-k-j: for each k
 * the row of B is added into an fp64 accumulator row.  Every acc[j] still
 * receives its K terms in ascending k, one rounding per addition, so each
 * acc[j] is bit-identical to the textbook dot product over k; only the memory
 * walk differs.  oracle_sgemm_entries() below is that textbook dot product,
 * and the test suite checks the two agree bit-for-bit.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - beta == 0 follows the literal formula (C is read and multiplied by 0).
 *  - K == 0 gives an empty sum, so C_out = round(beta * C_in).
 *  - Argument rules (checked before any work, BLAS-style negative codes that
 *    name the 1-based position of the first bad argument):
 *      M<0 -> -1, N<0 -> -2, K<0 -> -3,
 *      A==NULL while M>0 and K>0 -> -5,  lda < max(1,K) -> -6,
 *      B==NULL while K>0 and N>0 -> -7,  ldb < max(1,N) -> -8,
 *      C==NULL while M>0 and N>0 -> -10, ldc < max(1,N) -> -11.
 */
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int64_t max1(int64_t v) { return v > 1 ? v : 1; }

static int check_args(int64_t M, int64_t N, int64_t K, const float *A,
                      int64_t lda, const float *B, int64_t ldb, const float *C,
                      int64_t ldc) {
  if (M < 0) return -1;
  if (N < 0) return -2;
  if (K < 0) return -3;
  if (A == NULL && M > 0 && K > 0) return -5;
  if (lda < max1(K)) return -6;
  if (B == NULL && K > 0 && N > 0) return -7;
  if (ldb < max1(N)) return -8;
  if (C == NULL && M > 0 && N > 0) return -10;
  if (ldc < max1(N)) return -11;
  return 0;
}

/*
 * Full GEMM.  C is updated in place (fp32).  If C64 is not NULL, the fp64
 * value before the final rounding is also stored, C64[i*ldc64 + j], for the
 * tolerance test (ldc64 >= N).
 */
int oracle_sgemm(int64_t M, int64_t N, int64_t K, float alpha, const float *A,
                 int64_t lda, const float *B, int64_t ldb, float beta, float *C,
                 int64_t ldc, double *C64, int64_t ldc64) {
  int rc = check_args(M, N, K, A, lda, B, ldb, C, ldc);
  if (rc != 0) return rc;
  if (C64 != NULL && ldc64 < max1(N)) return -13;
  if (M == 0 || N == 0) return 0;

  int failed = 0;
#pragma omp parallel
  {
    double *acc = (double *)malloc((size_t)N * sizeof(double));
    if (acc == NULL) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
      if (acc == NULL) continue;
      for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const double a = (double)A[i * lda + k];
        const float *brow = B + k * ldb;
        for (int64_t j = 0; j < N; ++j) acc[j] += a * (double)brow[j];
      }
      for (int64_t j = 0; j < N; ++j) {
        const double v = (double)alpha * acc[j] + (double)beta * (double)C[i * ldc + j];
        if (C64 != NULL) C64[i * ldc64 + j] = v;
        C[i * ldc + j] = (float)v;
      }
    }
    free(acc);
  }
  return failed ? 100 : 0;
}

/*
 * Selected entries, each the textbook dot product over ascending k:
 *   out64[t] = alpha * sum_k A[rows[t],k]*B[k,cols[t]] + beta * Cin[rows[t],cols[t]]
 *   out32[t] = (float)out64[t]
 * Cin is only read.  Used where the full product is too large for the CPU.
 * Returns -20 if any requested (row, col) is outside M x N.
 */
int oracle_sgemm_entries(int64_t n, const int64_t *rows, const int64_t *cols,
                         int64_t M, int64_t N, int64_t K, float alpha,
                         const float *A, int64_t lda, const float *B,
                         int64_t ldb, float beta, const float *Cin, int64_t ldc,
                         float *out32, double *out64) {
  int rc = check_args(M, N, K, A, lda, B, ldb, Cin, ldc);
  if (rc != 0) return rc;
  for (int64_t t = 0; t < n; ++t)
    if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return -20;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n; ++t) {
    const int64_t i = rows[t], j = cols[t];
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k)
      s += (double)A[i * lda + k] * (double)B[k * ldb + j];
    const double v = (double)alpha * s + (double)beta * (double)Cin[i * ldc + j];
    if (out64 != NULL) out64[t] = v;
    if (out32 != NULL) out32[t] = (float)v;
  }
  return 0;
}

/* Threads the oracle may use (<= 0 leaves the OpenMP default). */
void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
