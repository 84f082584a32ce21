/*
 * CPU oracle for single-precision dense matrix multiply, C = A * B.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark load it.  It shares no code, header, table or
 * helper with the GPU library.
 *
 * What it computes (amittech.dev, "3.5 Project: tiled matrix multiplication",
 * section "starter scaffolding", the CPU reference routine): for row-major
 * operands, every output element is the dot product of a row of A with a
 * column of B, with every product formed in double precision from the two
 * float inputs and the sum accumulated in double precision in ascending k.
 * Unlike that routine, the sum is returned in double (not rounded back to
 * float) so that the checker can measure the GPU error against it; the
 * page's float-rounded value is simply (float) of what is returned here.
 *
 * Generalisation to M x K times K x N with leading dimensions: element
 * (r, c) of a row-major matrix with leading dimension ld lives at r*ld + c
 * (the same page, section "the numeric background", fixes row-major N x N
 * storage; BLAS leading-dimension convention supplies the rest).
 *
 * The bound matrix S[i][j] = sum_k |A[i][k] * B[k][j]| is the magnitude sum
 * that the componentwise forward error bound of a float dot product scales
 * with; it is computed by the same loop on |A| and |B|.
 *
 * Loop order is i-k-j with one double accumulator row per output row.  For
 * every single (i, j) the additions still happen in ascending k, so each
 * element is bit-identical to the page's i-j-k triple loop.  Every product
 * of two floats is exact in double (24 + 24 <= 53 significant bits).
 * Compile with -ffp-contract=off so that no multiply-add is fused.
 *
 * Rows are split over POSIX threads; each thread owns whole output rows, so
 * the result does not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* One output row: acc[j] = sum_k a[k] * b[k*ldb + j], and optionally the
 * magnitude sum s[j] = sum_k |a[k] * b[k*ldb + j]|, both in ascending k. */
static void oracle_row(int64_t N, int64_t K, const float *a, const float *B,
                       int64_t ldb, double *acc, double *s) {
    for (int64_t j = 0; j < N; j++) acc[j] = 0.0;
    if (s)
        for (int64_t j = 0; j < N; j++) s[j] = 0.0;
    for (int64_t k = 0; k < K; k++) {
        const double aik = (double)a[k];
        const float *brow = B + k * ldb;
        for (int64_t j = 0; j < N; j++) acc[j] += aik * (double)brow[j];
        if (s) {
            const double mag = fabs(aik);
            for (int64_t j = 0; j < N; j++) s[j] += mag * fabs((double)brow[j]);
        }
    }
}

typedef struct {
    int64_t N, K, lda, ldb, ldc;
    const float *A, *B;
    double *C, *S;
    const int64_t *rows; /* NULL: rows r0..r1-1 are output rows r0..r1-1 */
    int64_t r0, r1;
} row_job;

static void *row_worker(void *p) {
    row_job *j = (row_job *)p;
    for (int64_t r = j->r0; r < j->r1; r++) {
        const int64_t src = j->rows ? j->rows[r] : r;
        oracle_row(j->N, j->K, j->A + src * j->lda, j->B, j->ldb,
                   j->C + r * j->ldc, j->S ? j->S + r * j->ldc : NULL);
    }
    return NULL;
}

static void run_rows(int64_t nrows, const int64_t *rows, int64_t N, int64_t K,
                     const float *A, int64_t lda, const float *B, int64_t ldb,
                     double *C, double *S, int64_t ldc, int threads) {
    if (nrows <= 0) return;
    if (threads < 1) threads = 1;
    if (threads > nrows) threads = (int)nrows;
    row_job *jobs = (row_job *)calloc((size_t)threads, sizeof(row_job));
    pthread_t *tid = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    int64_t per = nrows / threads, extra = nrows % threads, r = 0;
    for (int t = 0; t < threads; t++) {
        int64_t cnt = per + (t < extra ? 1 : 0);
        row_job j = {N, K, lda, ldb, ldc, A, B, C, S, rows, r, r + cnt};
        jobs[t] = j;
        r += cnt;
    }
    for (int t = 1; t < threads; t++) pthread_create(&tid[t], NULL, row_worker, &jobs[t]);
    row_worker(&jobs[0]);
    for (int t = 1; t < threads; t++) pthread_join(tid[t], NULL);
    free(jobs);
    free(tid);
}

/* Full product.  C (and S when non-NULL) are M x N double, leading
 * dimension ldc.  Returns 0, or -1 on a negative size. */
int oracle_sgemm_f64(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                     const float *B, int64_t ldb, double *C, double *S, int64_t ldc,
                     int threads) {
    if (M < 0 || N < 0 || K < 0) return -1;
    run_rows(M, NULL, N, K, A, lda, B, ldb, C, S, ldc, threads);
    return 0;
}

/* Selected whole rows: output row t (of nrows) is row rows[t] of A*B. */
int oracle_sgemm_rows_f64(int64_t nrows, const int64_t *rows, int64_t N, int64_t K,
                          const float *A, int64_t lda, const float *B, int64_t ldb,
                          double *C, double *S, int64_t ldc, int threads) {
    if (nrows < 0 || N < 0 || K < 0) return -1;
    run_rows(nrows, rows, N, K, A, lda, B, ldb, C, S, ldc, threads);
    return 0;
}

/* Selected single elements (rows[t], cols[t]) as plain dot products in
 * ascending k; used where the full product is too large to form. */
int oracle_sgemm_entries_f64(int64_t count, const int64_t *rows, const int64_t *cols,
                             int64_t K, const float *A, int64_t lda, const float *B,
                             int64_t ldb, double *out, double *bound) {
    if (count < 0 || K < 0) return -1;
    for (int64_t t = 0; t < count; t++) {
        const float *a = A + rows[t] * lda;
        const float *b = B + cols[t];
        double acc = 0.0, s = 0.0;
        for (int64_t k = 0; k < K; k++) {
            const double p = (double)a[k] * (double)b[k * ldb];
            acc += p;
            s += fabs(p);
        }
        out[t] = acc;
        if (bound) bound[t] = s;
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * General form, row-major: C = alpha * op(A) * op(B) + beta * C0, the BLAS
 * operation of the course's library call (amittech.dev, "3.5 Project: tiled
 * matrix multiplication", section "the reference ceiling").  op(A) is M x K:
 * A itself (stored M x K) or, with transa, the transpose of A stored K x M;
 * op(B) is K x N likewise (stored K x N, or N x K with transb).  With
 * alpha == 0 or K == 0 the product is not formed; with beta == 0, C0 is not
 * read.  Also returned: S = |alpha| * sum_k |op(A)[i][k] op(B)[k][j]| and
 * E = |alpha * sum_k op(A)[i][k] op(B)[k][j]| + |beta * C0[i][j]|, the two
 * magnitudes the checker's bound scales with.  Plain element-by-element
 * loops, ascending k, in double.
 */
int oracle_sgemm_ex_f64(int transa, int transb, int64_t M, int64_t N, int64_t K, double alpha,
                        const float *A, int64_t lda, const float *B, int64_t ldb, double beta,
                        const float *C0, int64_t ldc0, double *C, double *S, double *E,
                        int64_t ldc) {
    if (M < 0 || N < 0 || K < 0) return -1;
    for (int64_t i = 0; i < M; i++)
        for (int64_t j = 0; j < N; j++) {
            double acc = 0.0, mag = 0.0;
            if (alpha != 0.0)
                for (int64_t k = 0; k < K; k++) {
                    const double a = transa ? (double)A[k * lda + i] : (double)A[i * lda + k];
                    const double b = transb ? (double)B[j * ldb + k] : (double)B[k * ldb + j];
                    acc += a * b;
                    mag += fabs(a * b);
                }
            const double c0 = beta != 0.0 ? beta * (double)C0[i * ldc0 + j] : 0.0;
            C[i * ldc + j] = alpha * acc + c0;
            S[i * ldc + j] = fabs(alpha) * mag;
            E[i * ldc + j] = fabs(alpha * acc) + fabs(c0);
        }
    return 0;
}

/* ------------------------------------------------------------------------
 * Compute-roof probes (amittech.dev, "7.3 Bandwidths and peak rate -
 * exercises", exercise 5).
 *
 * Chain probe: chain j (0 <= j < chains) starts at (j + 1) / 16 and is
 * updated iters times as acc = acc * x + y with a single rounding (fmaf),
 * which is what a fused multiply-add instruction computes.
 */
void oracle_fma_chain_f32(int64_t iters, float x, float y, int chains, float *out) {
    for (int j = 0; j < chains; j++) {
        float acc = 0.0625f * (float)(j + 1);
        for (int64_t i = 0; i < iters; i++) acc = fmaf(acc, x, y);
        out[j] = acc;
    }
}

/* Matrix-unit probe: the 32 x 32 result of adding the product of A (32 x 2,
 * A[i][k] = a_vals[i + 32 k]) and B (2 x 32, B[k][j] = b_vals[j + 32 k])
 * iters times, in double, row-major.  With small integer operands every
 * partial sum is exact in float too. */
void oracle_mfma_probe_f64(int64_t iters, const float *a_vals, const float *b_vals, double *D) {
    for (int i = 0; i < 32; i++)
        for (int j = 0; j < 32; j++) {
            double p = 0.0;
            for (int k = 0; k < 2; k++) p += (double)a_vals[i + 32 * k] * (double)b_vals[j + 32 * k];
            D[i * 32 + j] = (double)iters * p;
        }
}
