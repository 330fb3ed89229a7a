/*
 * Plain CPU reference SGEMM with FP64 accumulation.
 *
 * TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or run this library. It shares no
 * code, header, table or helper with the HIP library, and neither includes
 * nor links the other.
 *
 * What it computes, for row-major matrices and op in {N, T}:
 *
 *     C(i,j) <- alpha * sum_{k=0}^{K-1} opA(i,k) * opB(k,j) + beta * C(i,j)
 *
 * for 0 <= i < M, 0 <= j < N. This is the BLAS SGEMM operation
 * C = alpha*op(A)*op(B) + beta*C named in the overview of the itan.pw page on
 * SGEMM optimisation for the RTX 4090, with the row-major sum
 * C_ij = sum_k A_ik B_kj of the problem definition (问题定义) of
 * "【CUDA】Sgemm单精度矩阵乘法" (klklkl10086.github.io). That page's CPU
 * check (section 代码框架) is a plain triple loop accumulating in float; here
 * the sum is carried in double instead and rounded to float once, so this
 * result is the double-precision value alpha*s + beta*c rounded to nearest.
 *
 * Readings taken where the pages are silent:
 *   - opA(i,k) = A[i*lda + k] for 'N'/'n', A[k*lda + i] for 'T'/'t'/'C'/'c';
 *     opB(k,j) = B[k*ldb + j] for 'N', B[j*ldb + k] for 'T'; C(i,j) = C[i*ldc + j].
 *   - Each product of two floats is exact in double; the k sum runs in
 *     ascending k; alpha and beta are applied in double; one final
 *     round-to-nearest conversion to float.
 *   - beta == 0: C is not read (NaN in C does not propagate).
 *   - alpha == 0 or K == 0: A and B are not read; C <- beta*C (0 if beta == 0).
 *   - M == 0 or N == 0: nothing happens.
 *   - Argument errors follow BLAS info numbering (argument position, negated):
 *     -1 transA, -2 transB, -3 M, -4 N, -5 K, -7 A null, -8 lda, -9 B null,
 *     -10 ldb, -12 C null, -13 ldc.
 *
 * The loop order is i, k, j with one double accumulator per column of the
 * current row. Every (i, j) still sums its products in ascending k, so the
 * result is bit-identical to the i, j, k order; the j loop carries no
 * dependence, so the compiler may vectorise it without changing any sum.
 * Rows are split over OpenMP threads; each row is computed by one thread
 * exactly as above, so the result does not depend on the thread count.
 *
 * Build: gcc -O3 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math, no
 * FMA contraction).
 */
#include <stdlib.h>
#include <string.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int op_is_n(char t) { return t == 'N' || t == 'n'; }
static int op_is_t(char t) { return t == 'T' || t == 't' || t == 'C' || t == 'c'; }

static int check_args(char transA, char transB, int M, int N, int K, float alpha,
                      const float *A, int lda, const float *B, int ldb,
                      float beta, const float *C, int ldc)
{
    if (!op_is_n(transA) && !op_is_t(transA)) return -1;
    if (!op_is_n(transB) && !op_is_t(transB)) return -2;
    if (M < 0) return -3;
    if (N < 0) return -4;
    if (K < 0) return -5;
    int a_cols = op_is_n(transA) ? K : M;       /* stored A is M x K or K x M */
    int b_cols = op_is_n(transB) ? N : K;       /* stored B is K x N or N x K */
    if (lda < (a_cols > 1 ? a_cols : 1)) return -8;
    if (ldb < (b_cols > 1 ? b_cols : 1)) return -10;
    if (ldc < (N > 1 ? N : 1)) return -13;
    if (M == 0 || N == 0) return 0;
    int reads_ab = (alpha != 0.0f) && (K > 0);
    if (reads_ab && A == NULL) return -7;
    if (reads_ab && B == NULL) return -9;
    if (C == NULL) return -12;
    (void)beta;
    return 0;
}

static float opA(char transA, const float *A, int lda, int i, int k)
{
    return op_is_n(transA) ? A[(size_t)i * lda + k] : A[(size_t)k * lda + i];
}

static float opB(char transB, const float *B, int ldb, int k, int j)
{
    return op_is_n(transB) ? B[(size_t)k * ldb + j] : B[(size_t)j * ldb + k];
}

/* One output from its own sum; used for both the full product and samples. */
static float one_entry(char transA, char transB, int K, float alpha,
                       const float *A, int lda, const float *B, int ldb,
                       float beta, float c_in, int i, int j)
{
    double s = 0.0;
    if (alpha != 0.0f) {
        for (int k = 0; k < K; ++k)
            s += (double)opA(transA, A, lda, i, k) * (double)opB(transB, B, ldb, k, j);
    }
    double t = (beta == 0.0f) ? 0.0 : (double)beta * (double)c_in;
    double r = (alpha == 0.0f) ? t : (double)alpha * s + t;
    return (float)r;
}

int oracle_sgemm(char transA, char transB, int M, int N, int K, float alpha,
                 const float *A, int lda, const float *B, int ldb,
                 float beta, float *C, int ldc)
{
    int rc = check_args(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
    if (rc != 0 || M == 0 || N == 0) return rc;

    if (alpha == 0.0f || K == 0) {
        for (int i = 0; i < M; ++i)
            for (int j = 0; j < N; ++j) {
                float *c = &C[(size_t)i * ldc + j];
                *c = (beta == 0.0f) ? 0.0f : (float)((double)beta * (double)*c);
            }
        return 0;
    }

    /* opB gathered once as a K x N row-major float matrix (a copy, no arithmetic). */
    float *Bop = (float *)malloc((size_t)K * N * sizeof(float));
    if (Bop == NULL) return 2;
    for (int k = 0; k < K; ++k)
        for (int j = 0; j < N; ++j)
            Bop[(size_t)k * N + j] = opB(transB, B, ldb, k, j);

    int fail = 0;
#pragma omp parallel
    {
        double *acc = (double *)malloc((size_t)N * sizeof(double));
        if (acc == NULL) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(static)
        for (int i = 0; i < M; ++i) {
            if (acc == NULL) continue;
            for (int j = 0; j < N; ++j) acc[j] = 0.0;
            for (int k = 0; k < K; ++k) {
                const double a = (double)opA(transA, A, lda, i, k);
                const float *brow = &Bop[(size_t)k * N];
                for (int j = 0; j < N; ++j) acc[j] += a * (double)brow[j];
            }
            float *crow = &C[(size_t)i * ldc];
            for (int j = 0; j < N; ++j) {
                double t = (beta == 0.0f) ? 0.0 : (double)beta * (double)crow[j];
                crow[j] = (float)((double)alpha * acc[j] + t);
            }
        }
        free(acc);
    }
    free(Bop);
    return fail ? 2 : 0;
}

/*
 * The same result for a list of (row, col) positions only, each computed on
 * its own by the single-entry sum above; out[p] receives C_out(rows[p], cols[p])
 * given c_in[p] = C_in(rows[p], cols[p]). Used to check outputs at sizes where
 * the full product would take too long on the host.
 */
int oracle_sgemm_entries(char transA, char transB, int M, int N, int K, float alpha,
                         const float *A, int lda, const float *B, int ldb,
                         float beta, const float *c_in, int count,
                         const int *rows, const int *cols, float *out)
{
    int rc = check_args(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta,
                        (const float *)out, N > 1 ? N : 1);
    if (rc != 0) return rc;
    if (beta != 0.0f && c_in == NULL && count > 0) return -12;
    for (int p = 0; p < count; ++p)
        if (rows[p] < 0 || rows[p] >= M || cols[p] < 0 || cols[p] >= N) return -14;
#pragma omp parallel for schedule(static)
    for (int p = 0; p < count; ++p)
        out[p] = one_entry(transA, transB, K, alpha, A, lda, B, ldb, beta,
                           c_in ? c_in[p] : 0.0f, rows[p], cols[p]);
    return 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
