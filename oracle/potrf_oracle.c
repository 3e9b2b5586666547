/*
 * CPU oracle for batched Cholesky (potrf) and the positive-definite solve
 * (posv).  TEST INFRASTRUCTURE ONLY: nothing on the product path may link,
 * load or call this file.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header or table
 * with the HIP library.
 *
 * What it computes (BatchLAS documentation, page "Batched Cholesky (potrf)
 * and the fused positive-definite solve (posv)"):
 *   - potrf factors each Hermitian positive-definite matrix of a batch as
 *     A = L L^H (Lower) or A = U^H U (Upper); Upper is the same recurrence run
 *     on S(i,c) = conj(A(c,i)), i.e. a load/store transform
 *     (section "Selection", paragraph on can_run() terms; section
 *     "The shared tiny-tier invariants").
 *   - info[b] = 0 on success, else the 1-based column of the first Schur
 *     pivot d that fails d > 0; later failures never overwrite it
 *     (section "potrf: correctness findings", item 6; section
 *     "Armed breaks (R9) - LPanel", break 5, where the pivot test is
 *     bad = ok && !(d > 0), so zero, negative and NaN pivots all fail).
 *   - posv factors A, then solves L y = b and L^H x = y for each right-hand
 *     side (section "The fused posv tier"; section "The fused potrs solve").
 *
 * The factor of a Hermitian positive-definite matrix is unique, so this file
 * writes out that definition with the textbook unblocked column (left-looking,
 * xPOTF2-order) algorithm:
 *     for j = 0..n-1:
 *         d      = Re A(j,j) - sum_{p<j} |L(j,p)|^2          (p ascending)
 *         if !(d > 0): info = j+1, stop this matrix
 *         L(j,j) = sqrt(d)
 *         L(i,j) = (A(i,j) - sum_{p<j} L(i,p) conj(L(j,p))) / L(j,j),  i > j
 * Arithmetic is in the storage precision (float for float and complex-float,
 * double for the double types), compiled without FMA contraction or
 * fast-math, so the result is reproducible at any thread count: the batch is
 * split across threads and each matrix is sequential.
 *
 * Readings taken where the pages are silent:
 *   - the imaginary part of a complex diagonal is ignored on input, and the
 *     output diagonal is written with imaginary part +0;
 *   - after a failure at column j, columns 0..j-1 hold L, A(j,j) holds the
 *     failing Schur value d, and nothing else is written (LAPACK's xPOTF2);
 *   - posv leaves B unchanged for an item whose info is nonzero;
 *   - the other triangle and all padding are neither read nor written.
 *
 * Complex products are written out by hand as real multiplies and adds.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

enum { OR_F32 = 0, OR_F64 = 1, OR_C64 = 2, OR_C128 = 3 };
enum { OR_LOWER = 0, OR_UPPER = 1 };

typedef struct { float re, im; } or_c64;
typedef struct { double re, im; } or_c128;

/* ------------------------------------------------------------------------ */
/* Real element types.  S(i,c), i >= c, is A(i,c) for Lower and A(c,i) for    */
/* Upper (conj is the identity for real numbers).                              */
/* ------------------------------------------------------------------------ */
#define OR_REAL_KERNELS(R, SUF, SQRT)                                                 \
static inline R *s_at_##SUF(R *A, int64_t lda, int upper, int64_t i, int64_t c) \
{                                                                               \
    return upper ? &A[c + i * lda] : &A[i + c * lda];                           \
}                                                                               \
                                                                                \
static int32_t factor_##SUF(R *A, int64_t lda, int upper, int64_t n)           \
{                                                                               \
    for (int64_t j = 0; j < n; ++j) {                                           \
        R s = 0;                                                                \
        for (int64_t p = 0; p < j; ++p) {                                       \
            R l = *s_at_##SUF(A, lda, upper, j, p);                             \
            s += l * l;                                                         \
        }                                                                       \
        R d = *s_at_##SUF(A, lda, upper, j, j) - s;                             \
        if (!(d > 0)) {                                                         \
            *s_at_##SUF(A, lda, upper, j, j) = d;                               \
            return (int32_t)(j + 1);                                            \
        }                                                                       \
        R ljj = SQRT(d);                                                        \
        *s_at_##SUF(A, lda, upper, j, j) = ljj;                                 \
        for (int64_t i = j + 1; i < n; ++i) {                                   \
            R t = *s_at_##SUF(A, lda, upper, i, j);                             \
            for (int64_t p = 0; p < j; ++p)                                     \
                t -= *s_at_##SUF(A, lda, upper, i, p) *                         \
                     *s_at_##SUF(A, lda, upper, j, p);                          \
            *s_at_##SUF(A, lda, upper, i, j) = t / ljj;                         \
        }                                                                       \
    }                                                                           \
    return 0;                                                                   \
}                                                                               \
                                                                                \
/* Solve (L L^H) x = b in place for nrhs columns, L from the factored S. */    \
static void solve_##SUF(const R *A, int64_t lda, int upper, int64_t n,          \
                        int64_t nrhs, R *B, int64_t ldb)                        \
{                                                                               \
    R *Am = (R *)A;                                                             \
    for (int64_t r = 0; r < nrhs; ++r) {                                        \
        R *b = B + r * ldb;                                                     \
        for (int64_t i = 0; i < n; ++i) {          /* forward: L y = b   */     \
            R t = b[i];                                                         \
            for (int64_t p = 0; p < i; ++p)                                     \
                t -= *s_at_##SUF(Am, lda, upper, i, p) * b[p];                  \
            b[i] = t / *s_at_##SUF(Am, lda, upper, i, i);                       \
        }                                                                       \
        for (int64_t i = n - 1; i >= 0; --i) {     /* backward: L^H x = y */    \
            R t = b[i];                                                         \
            for (int64_t p = i + 1; p < n; ++p)                                 \
                t -= *s_at_##SUF(Am, lda, upper, p, i) * b[p];                  \
            b[i] = t / *s_at_##SUF(Am, lda, upper, i, i);                       \
        }                                                                       \
    }                                                                           \
}

OR_REAL_KERNELS(float, f32, sqrtf)
OR_REAL_KERNELS(double, f64, sqrt)

/* ------------------------------------------------------------------------ */
/* Complex element types.  S(i,c) = A(i,c) for Lower, conj(A(c,i)) for Upper. */
/* ------------------------------------------------------------------------ */
#define OR_CPLX_KERNELS(C, R, SUF, SQRT)                                        \
static inline C s_get_##SUF(const C *A, int64_t lda, int upper, int64_t i,      \
                            int64_t c)                                          \
{                                                                               \
    C v;                                                                        \
    if (upper) { v = A[c + i * lda]; v.im = -v.im; }                            \
    else       { v = A[i + c * lda]; }                                          \
    return v;                                                                   \
}                                                                               \
static inline void s_put_##SUF(C *A, int64_t lda, int upper, int64_t i,         \
                               int64_t c, C v)                                  \
{                                                                               \
    if (upper) { v.im = -v.im; A[c + i * lda] = v; }                            \
    else       { A[i + c * lda] = v; }                                          \
}                                                                               \
                                                                                \
static int32_t factor_##SUF(C *A, int64_t lda, int upper, int64_t n)           \
{                                                                               \
    for (int64_t j = 0; j < n; ++j) {                                           \
        R s = 0;                                                                \
        for (int64_t p = 0; p < j; ++p) {                                       \
            C l = s_get_##SUF(A, lda, upper, j, p);                             \
            s += l.re * l.re + l.im * l.im;                                     \
        }                                                                       \
        R d = s_get_##SUF(A, lda, upper, j, j).re - s;                          \
        if (!(d > 0)) {                                                         \
            A[j + j * lda].re = d;         /* diagonal: same cell either uplo */\
            A[j + j * lda].im = 0;                                              \
            return (int32_t)(j + 1);                                            \
        }                                                                       \
        R ljj = SQRT(d);                                                        \
        A[j + j * lda].re = ljj;           /* imaginary part written as +0   */ \
        A[j + j * lda].im = 0;                                                  \
        for (int64_t i = j + 1; i < n; ++i) {                                   \
            C t = s_get_##SUF(A, lda, upper, i, j);                             \
            for (int64_t p = 0; p < j; ++p) {                                   \
                C a = s_get_##SUF(A, lda, upper, i, p);  /* L(i,p)      */      \
                C b = s_get_##SUF(A, lda, upper, j, p);  /* L(j,p)      */      \
                /* t -= a * conj(b) = (a.re b.re + a.im b.im)              */   \
                /*                  + i (a.im b.re - a.re b.im)            */   \
                t.re -= a.re * b.re + a.im * b.im;                              \
                t.im -= a.im * b.re - a.re * b.im;                              \
            }                                                                   \
            t.re = t.re / ljj;                                                  \
            t.im = t.im / ljj;                                                  \
            s_put_##SUF(A, lda, upper, i, j, t);                                \
        }                                                                       \
    }                                                                           \
    return 0;                                                                   \
}                                                                               \
                                                                                \
static void solve_##SUF(const C *A, int64_t lda, int upper, int64_t n,          \
                        int64_t nrhs, C *B, int64_t ldb)                        \
{                                                                               \
    for (int64_t r = 0; r < nrhs; ++r) {                                        \
        C *b = B + r * ldb;                                                     \
        for (int64_t i = 0; i < n; ++i) {          /* forward: L y = b   */     \
            C t = b[i];                                                         \
            for (int64_t p = 0; p < i; ++p) {                                   \
                C l = s_get_##SUF(A, lda, upper, i, p);  /* L(i,p)      */      \
                C y = b[p];                                                     \
                t.re -= l.re * y.re - l.im * y.im;                              \
                t.im -= l.re * y.im + l.im * y.re;                              \
            }                                                                   \
            R dg = s_get_##SUF(A, lda, upper, i, i).re;                         \
            b[i].re = t.re / dg;                                                \
            b[i].im = t.im / dg;                                                \
        }                                                                       \
        for (int64_t i = n - 1; i >= 0; --i) {     /* backward: L^H x = y */    \
            C t = b[i];                                                         \
            for (int64_t p = i + 1; p < n; ++p) {                               \
                C l = s_get_##SUF(A, lda, upper, p, i);  /* L(p,i)      */      \
                C x = b[p];                                                     \
                /* t -= conj(l) * x */                                          \
                t.re -= l.re * x.re + l.im * x.im;                              \
                t.im -= l.re * x.im - l.im * x.re;                              \
            }                                                                   \
            R dg = s_get_##SUF(A, lda, upper, i, i).re;                         \
            b[i].re = t.re / dg;                                                \
            b[i].im = t.im / dg;                                                \
        }                                                                       \
    }                                                                           \
}

OR_CPLX_KERNELS(or_c64, float, c64, sqrtf)
OR_CPLX_KERNELS(or_c128, double, c128, sqrt)

/* ------------------------------------------------------------------------ */
/* Batch driver: static contiguous split of the batch over threads.           */
/* ------------------------------------------------------------------------ */
typedef struct {
    int dtype, uplo;
    int64_t n, nrhs;
    void *A; int64_t lda, strideA;
    void *B; int64_t ldb, strideB;
    int32_t *info;
    int64_t b0, b1;
} or_job;

static size_t elem_size(int dtype)
{
    switch (dtype) {
    case OR_F32: return 4;
    case OR_F64: return 8;
    case OR_C64: return 8;
    case OR_C128: return 16;
    }
    return 0;
}

static void *run_job(void *arg)
{
    or_job *jb = (or_job *)arg;
    size_t es = elem_size(jb->dtype);
    for (int64_t b = jb->b0; b < jb->b1; ++b) {
        char *a = (char *)jb->A + (size_t)b * (size_t)jb->strideA * es;
        char *x = jb->B ? (char *)jb->B + (size_t)b * (size_t)jb->strideB * es : NULL;
        int32_t inf = 0;
        switch (jb->dtype) {
        case OR_F32:
            inf = factor_f32((float *)a, jb->lda, jb->uplo, jb->n);
            if (x && inf == 0) solve_f32((float *)a, jb->lda, jb->uplo, jb->n, jb->nrhs, (float *)x, jb->ldb);
            break;
        case OR_F64:
            inf = factor_f64((double *)a, jb->lda, jb->uplo, jb->n);
            if (x && inf == 0) solve_f64((double *)a, jb->lda, jb->uplo, jb->n, jb->nrhs, (double *)x, jb->ldb);
            break;
        case OR_C64:
            inf = factor_c64((or_c64 *)a, jb->lda, jb->uplo, jb->n);
            if (x && inf == 0) solve_c64((or_c64 *)a, jb->lda, jb->uplo, jb->n, jb->nrhs, (or_c64 *)x, jb->ldb);
            break;
        case OR_C128:
            inf = factor_c128((or_c128 *)a, jb->lda, jb->uplo, jb->n);
            if (x && inf == 0) solve_c128((or_c128 *)a, jb->lda, jb->uplo, jb->n, jb->nrhs, (or_c128 *)x, jb->ldb);
            break;
        }
        if (jb->info) jb->info[b] = inf;
    }
    return NULL;
}

static int run_batch(or_job proto, int64_t batch, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if ((int64_t)nthreads > batch) nthreads = (int)batch;
    if (nthreads == 1) {
        proto.b0 = 0; proto.b1 = batch;
        run_job(&proto);
        return 0;
    }
    or_job *jobs = (or_job *)malloc(sizeof(or_job) * (size_t)nthreads);
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!jobs || !tid) { free(jobs); free(tid); return -2; }
    int64_t per = batch / nthreads, rem = batch % nthreads, start = 0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t cnt = per + (t < rem ? 1 : 0);
        jobs[t] = proto;
        jobs[t].b0 = start; jobs[t].b1 = start + cnt;
        start += cnt;
        if (pthread_create(&tid[t], NULL, run_job, &jobs[t]) != 0) {
            run_job(&jobs[t]);            /* run inline if no thread */
            tid[t] = 0;
        }
    }
    for (int t = 0; t < nthreads; ++t)
        if (tid[t]) pthread_join(tid[t], NULL);
    free(jobs); free(tid);
    return 0;
}

/* Returns 0 on success, -1 on an invalid argument. */
int oracle_potrf(int dtype, int uplo, int64_t n, void *A, int64_t lda,
                 int64_t strideA, int64_t batch, int32_t *info, int nthreads)
{
    if (elem_size(dtype) == 0 || (uplo != OR_LOWER && uplo != OR_UPPER)) return -1;
    if (n < 1 || batch < 1 || lda < n || strideA < lda * n || !A) return -1;
    or_job proto = { dtype, uplo, n, 0, A, lda, strideA, NULL, 0, 0, info, 0, 0 };
    return run_batch(proto, batch, nthreads);
}

int oracle_posv(int dtype, int uplo, int64_t n, int64_t nrhs, void *A,
                int64_t lda, int64_t strideA, void *B, int64_t ldb,
                int64_t strideB, int64_t batch, int32_t *info, int nthreads)
{
    if (elem_size(dtype) == 0 || (uplo != OR_LOWER && uplo != OR_UPPER)) return -1;
    if (n < 1 || nrhs < 1 || batch < 1 || lda < n || ldb < n) return -1;
    if (strideA < lda * n || strideB < ldb * nrhs || !A || !B) return -1;
    or_job proto = { dtype, uplo, n, nrhs, A, lda, strideA, B, ldb, strideB, info, 0, 0 };
    return run_batch(proto, batch, nthreads);
}
