/* Plain float64 GEMM accumulation for the CPU oracle. TEST INFRASTRUCTURE ONLY.
 *
 * acc[m][n] = sum over k = 0, 1, ..., K-1 (in that order) of a[m][k] * b[k][n]
 *
 * The GEMM definition of the first DeepGEMM page (sec. 1.1), written as the
 * textbook i-k-j triple loop: for each output row m, for each k, row k of b
 * scaled by a[m][k] is added into row m of acc. Every acc[m][n] is therefore
 * the float64 sum of its K products taken in ascending k. No blocking, no
 * reassociation: the compiler is told not to contract a*b+c into a fused
 * multiply-add (-ffp-contract=off) and not to reorder floating-point sums
 * (no -ffast-math). The only parallelism is over output rows, each row being
 * summed by one thread exactly as above.
 *
 * Operands are dense row-major float64 arrays (a: M x K, b: K x N, acc:
 * M x N), already decoded from their storage formats by the Python side.
 */
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

__attribute__((target_clones("avx2", "default")))
static void row_ikj(int64_t N, int64_t K, const double* arow, const double* b, double* crow) {
  memset(crow, 0, (size_t)N * sizeof(double));
  for (int64_t k = 0; k < K; ++k) {
    const double aik = arow[k];
    const double* brow = b + k * N;
    for (int64_t n = 0; n < N; ++n) crow[n] = crow[n] + aik * brow[n];
  }
}

/* threads <= 0: OpenMP's default team size. Returns the team size used. */
int oracle_gemm_f64(int64_t M, int64_t N, int64_t K, const double* a, const double* b,
                    double* acc, int threads) {
  int used = 1;
#ifdef _OPENMP
  const int team = threads > 0 ? threads : omp_get_max_threads();
#pragma omp parallel num_threads(team) if (M > 1)
  {
#pragma omp single
    used = omp_get_num_threads();
#pragma omp for schedule(static)
    for (int64_t m = 0; m < M; ++m) row_ikj(N, K, a + m * K, b, acc + m * N);
  }
#else
  (void)threads;
  for (int64_t m = 0; m < M; ++m) row_ikj(N, K, a + m * K, b, acc + m * N);
#endif
  return used;
}
