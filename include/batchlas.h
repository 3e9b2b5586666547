/*
 * batchlas -- batched Cholesky factorisation (potrf) and positive-definite
 * solve (posv) for many small independent Hermitian positive-definite
 * matrices, on AMD Instinct MI355X (gfx950).
 *
 * The operations are the ones described on the BatchLAS documentation's
 * perf_potrf page:
 *   potrf  factors every matrix of a batch as A = L L^H (Lower) or
 *          A = U^H U (Upper); Upper is the same recurrence applied to
 *          S(i,c) = conj(A(c,i)) (section "Selection", can_run() terms);
 *   posv   factors A and then solves A X = B with a forward solve L y = b and
 *          a backward solve L^H x = y per right-hand side (sections "posv
 *          selection", "The fused posv tier", "The fused potrs solve").
 * Per-matrix failure is reported through info, with the first failing
 * column winning (section "potrf: correctness findings", item 6).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory   All array pointers are DEVICE pointers owned by the caller.  The
 *          library allocates nothing persistent, keeps no pointer after it
 *          returns and makes no host<->device copy of its own.
 * Layout   Column-major.  Matrix b's element (i, c) is at
 *          A[b * strideA + c * lda + i].  lda, ldb and the strides count
 *          ELEMENTS and are 64-bit.  Complex elements are interleaved
 *          (re, im) pairs of the real type.  Matrices must not overlap
 *          (strideA >= lda * n).
 * Effects  potrf overwrites the referenced triangle of each A with L (Lower)
 *          or U (Upper); the diagonal is real and positive, with imaginary
 *          part +0.  The other triangle and all padding are neither read nor
 *          written.  posv also overwrites B with X for every item whose info
 *          is 0 and leaves B unchanged for an item whose info is nonzero.
 *          The imaginary part of an input diagonal is ignored.
 * info     int32[batch] device array: 0 on success, else the 1-based column
 *          of the first Schur pivot d with !(d > 0) (zero, negative and NaN
 *          pivots fail); a later failure never overwrites it.  For a failed
 *          item the leading info-1 columns hold the factor of the leading
 *          block; the rest of the referenced triangle is unspecified.  info
 *          may be NULL, in which case nothing is written.
 * Errors   Arguments are checked synchronously, before anything is enqueued
 *          and with no writes, in this order: n, nrhs, batch >= 1; lda, ldb
 *          >= n; strideA >= lda*n, strideB >= ldb*nrhs; non-null A (and B);
 *          dtype and uplo valid; the route runnable.  Numerical failure is
 *          never a status: it is reported only through info.  No C++
 *          exception crosses this interface.
 * Streams  Work is enqueued on `stream` (a hipStream_t; NULL is the default
 *          stream) with no internal synchronisation: results are valid once
 *          the stream has been synchronised.  The environment (route pins,
 *          trace) is read once, at the first call; there is no other global
 *          state, so calls from several host threads are safe.
 */
#ifndef BATCHLAS_H
#define BATCHLAS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same underlying type as hipStream_t, so a hipStream_t converts implicitly. */
typedef struct ihipStream_t *batchlas_stream_t;

typedef enum { BATCHLAS_LOWER = 0, BATCHLAS_UPPER = 1 } batchlas_uplo;

typedef enum {
    BATCHLAS_F32 = 0,   /* float                    */
    BATCHLAS_F64 = 1,   /* double                   */
    BATCHLAS_C64 = 2,   /* complex float  (re, im)  */
    BATCHLAS_C128 = 3   /* complex double (re, im)  */
} batchlas_dtype;

typedef enum {
    BATCHLAS_OK = 0,
    BATCHLAS_INVALID_VALUE = 1,   /* a size, leading dimension, stride, dtype or uplo is out of range */
    BATCHLAS_NULL_POINTER = 2,    /* A (or B) is NULL                                               */
    BATCHLAS_NOT_SUPPORTED = 3,   /* no kernel family serves this shape / the pinned family cannot   */
    BATCHLAS_HIP_ERROR = 4,       /* the HIP runtime reported an error while enqueueing              */
    BATCHLAS_INTERNAL = 5         /* an internal invariant failed                                    */
} batchlas_status;

/* Kernel families (the route).  AUTO lets the size dispatcher choose. */
typedef enum {
    BATCHLAS_FAMILY_AUTO = 0,
    BATCHLAS_FAMILY_TINY = 1,       /* registers, several matrices per wavefront          */
    BATCHLAS_FAMILY_LDS = 2,        /* one workgroup per matrix, matrix staged in LDS      */
    BATCHLAS_FAMILY_BLOCKED = 3,    /* panel factor + solve, MFMA trailing rank-k update   */
    BATCHLAS_FAMILY_POSV_TINY = 4,  /* fused factor + both solves in registers (posv only) */
    BATCHLAS_FAMILY_POSV_SPLIT = 5  /* potrf by any family, then a fused two-solve kernel  */
} batchlas_family;

/* Launch geometry chosen for a call (for tests and tracing). */
typedef struct {
    int32_t family;             /* batchlas_family actually used                         */
    int32_t lanes_per_matrix;   /* tiny / posv: lanes that share one matrix (P); in the
                                   wide fp32 window (orders 65..192) the workgroup         */
    int32_t rows_per_lane;      /* tiny / posv: rows each lane holds (R)                  */
    int32_t matrices_per_wave;  /* tiny / posv: matrices packed in one wavefront (G); 1
                                   in the wide window (one matrix per workgroup)           */
    int32_t block_threads;      /* threads per workgroup of the main kernel              */
    int32_t panel;              /* lds / blocked: panel width (nb); wide fp32 tiles: their
                                   column count; 0 otherwise                               */
    int64_t grid;               /* workgroups of the main kernel (first launch)          */
    int64_t lds_bytes;          /* LDS per workgroup of the main kernel                   */
} batchlas_route_info;

/*
 * potrf: factor `batch` Hermitian positive-definite n x n matrices in place.
 *   dt, uplo   element type; which triangle is referenced and overwritten
 *   n          order, >= 1
 *   A          device pointer to the first matrix (see Layout)
 *   lda        leading dimension in elements, >= n
 *   strideA    distance between consecutive matrices in elements, >= lda*n
 *   batch      number of matrices, >= 1
 *   info       device int32[batch] or NULL (see info)
 *   stream     HIP stream for the work
 * Returns BATCHLAS_OK once the work is enqueued.
 */
batchlas_status batchlas_potrf(batchlas_dtype dt, batchlas_uplo uplo, int64_t n,
                               void *A, int64_t lda, int64_t strideA, int64_t batch,
                               int32_t *info, batchlas_stream_t stream);

/*
 * posv: factor each A as potrf does, then solve A X = B for nrhs right-hand
 * sides per item, overwriting B with X.
 *   B          device pointer, n x nrhs per item, column-major
 *   ldb        >= n;  strideB >= ldb * nrhs
 * Other arguments as for batchlas_potrf.  A is overwritten with the factor.
 * Small orders with nrhs <= 4 run fused in one kernel (POSV_TINY); every
 * other shape that potrf serves runs as potrf followed by one kernel for both
 * triangular solves (POSV_SPLIT), which also keeps B of failed items when
 * info is NULL (it reads the failure off the factor's diagonal).
 */
batchlas_status batchlas_posv(batchlas_dtype dt, batchlas_uplo uplo, int64_t n, int64_t nrhs,
                              void *A, int64_t lda, int64_t strideA,
                              void *B, int64_t ldb, int64_t strideB, int64_t batch,
                              int32_t *info, batchlas_stream_t stream);

/*
 * Same operations with an explicit family instead of the dispatcher's choice
 * (or the environment pin).  A family that cannot run the shape returns
 * BATCHLAS_NOT_SUPPORTED before anything is enqueued.
 */
batchlas_status batchlas_potrf_family(batchlas_family family, batchlas_dtype dt,
                                      batchlas_uplo uplo, int64_t n, void *A, int64_t lda,
                                      int64_t strideA, int64_t batch, int32_t *info,
                                      batchlas_stream_t stream);
batchlas_status batchlas_posv_family(batchlas_family family, batchlas_dtype dt,
                                     batchlas_uplo uplo, int64_t n, int64_t nrhs,
                                     void *A, int64_t lda, int64_t strideA,
                                     void *B, int64_t ldb, int64_t strideB, int64_t batch,
                                     int32_t *info, batchlas_stream_t stream);

/* Typed wrappers (s = float, d = double, c = complex float, z = complex double). */
batchlas_status batchlas_spotrf(batchlas_uplo uplo, int64_t n, float *A, int64_t lda,
                                int64_t strideA, int64_t batch, int32_t *info,
                                batchlas_stream_t stream);
batchlas_status batchlas_dpotrf(batchlas_uplo uplo, int64_t n, double *A, int64_t lda,
                                int64_t strideA, int64_t batch, int32_t *info,
                                batchlas_stream_t stream);
batchlas_status batchlas_cpotrf(batchlas_uplo uplo, int64_t n, void *A, int64_t lda,
                                int64_t strideA, int64_t batch, int32_t *info,
                                batchlas_stream_t stream);
batchlas_status batchlas_zpotrf(batchlas_uplo uplo, int64_t n, void *A, int64_t lda,
                                int64_t strideA, int64_t batch, int32_t *info,
                                batchlas_stream_t stream);
batchlas_status batchlas_sposv(batchlas_uplo uplo, int64_t n, int64_t nrhs, float *A,
                               int64_t lda, int64_t strideA, float *B, int64_t ldb,
                               int64_t strideB, int64_t batch, int32_t *info,
                               batchlas_stream_t stream);
batchlas_status batchlas_dposv(batchlas_uplo uplo, int64_t n, int64_t nrhs, double *A,
                               int64_t lda, int64_t strideA, double *B, int64_t ldb,
                               int64_t strideB, int64_t batch, int32_t *info,
                               batchlas_stream_t stream);
batchlas_status batchlas_cposv(batchlas_uplo uplo, int64_t n, int64_t nrhs, void *A,
                               int64_t lda, int64_t strideA, void *B, int64_t ldb,
                               int64_t strideB, int64_t batch, int32_t *info,
                               batchlas_stream_t stream);
batchlas_status batchlas_zposv(batchlas_uplo uplo, int64_t n, int64_t nrhs, void *A,
                               int64_t lda, int64_t strideA, void *B, int64_t ldb,
                               int64_t strideB, int64_t batch, int32_t *info,
                               batchlas_stream_t stream);

/*
 * Route query: the family and launch geometry a call with these arguments
 * would use (nrhs = 0 asks about potrf, nrhs >= 1 about posv).  `family`
 * pins a family as in the *_family entry points; AUTO applies the dispatcher
 * and the environment pin.  Host-only: makes no HIP call.  Validates its
 * arguments like the operation would (pointers are not checked).
 */
batchlas_status batchlas_route(batchlas_family family, batchlas_dtype dt, batchlas_uplo uplo,
                               int64_t n, int64_t nrhs, int64_t lda, int64_t strideA,
                               int64_t batch, batchlas_route_info *out);

/* Static text for a status code. */
const char *batchlas_status_string(batchlas_status s);

/* The message of the last failing call made by this host thread ("" if none). */
const char *batchlas_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t batchlas_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BATCHLAS_H */
