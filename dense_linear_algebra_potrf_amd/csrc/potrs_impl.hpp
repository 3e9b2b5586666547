// Triangular solves with an already factored A (the split posv route):
// for each item, A X = B is solved as L Y = B, then L^H X = Y, with L the
// factor that potrf left in A (L itself for Lower; L = U^H for Upper, so
// L(i, j) = conj(A(j, i))).
//
// Prior art: the BatchLAS perf_potrf page, sections "posv selection" and "The
// fused potrs solve" (both solves in one launch over a batch of factored
// matrices).  Built for CDNA4 as follows: one workgroup takes one item and up
// to RC right-hand sides (a second grid dimension covers the rest), keeps
// those columns of B in LDS for both solves, and works in blocks of NBS rows:
// one wavefront solves the NBS x NBS diagonal block (lane i owns row i; the
// solved entry of a step is exchanged through LDS), then every thread
// updates the rows outside the block with the block's solved entries.  The
// factor is read from memory where it is used (column j of L is contiguous for
// Lower, so the row updates of the forward solve are coalesced).
//
// Failed items (info != 0) keep B unchanged.  With info == NULL the failure is
// read off the factor: potrf leaves a diagonal entry that is not > 0 (the
// square root of a pivot that is not > 0 is NaN or 0) exactly when it
// reports a failure.
#pragma once

#include "families.hpp"

namespace bl {
namespace potrs_detail {

constexpr int NBS = 32;          // rows per diagonal block
constexpr int THREADS = 256;
constexpr int RC = 4;            // right-hand sides per workgroup
constexpr int MAXN = 512;

template <typename T, bool UPPER>
__device__ __forceinline__ T lval(const T* __restrict__ Ab, int64_t lda, int i, int j) {
    if constexpr (UPPER) return conj(Ab[int64_t(i) * lda + j]);
    else return Ab[int64_t(j) * lda + i];
}

template <typename T, bool UPPER>
__global__ __launch_bounds__(THREADS) void potrs_kernel(
    const T* __restrict__ A, int n, int64_t lda, int64_t strideA, T* __restrict__ B, int nrhs,
    int64_t ldb, int64_t strideB, int64_t batch, const int32_t* __restrict__ info)
{
    using Rt = typename Traits<T>::R;
    __shared__ T X[MAXN * RC];            // X[i * RC + r]: row i, right-hand side r0 + r
    const int t = threadIdx.x;
    const int64_t b = blockIdx.x;
    const int r0 = blockIdx.y * RC;
    const int nr = min(RC, nrhs - r0);
    const T* __restrict__ Ab = A + b * strideA;
    T* __restrict__ Bb = B + b * strideB;

    // ---- failed items keep B
    int ok = 1;
    if (info != nullptr) {
        ok = info[b] == 0;
    } else {
        for (int i = t; i < n; i += THREADS) ok &= re(Ab[int64_t(i) * lda + i]) > Rt(0);
    }
    if (!__syncthreads_and(ok)) return;

    for (int idx = t; idx < n * RC; idx += THREADS) {
        const int i = idx % n, r = idx / n;
        X[i * RC + r] = r < nr ? Bb[int64_t(r0 + r) * ldb + i] : zero<T>();
    }
    __syncthreads();

    const int lane = t & 63;
    const int li = lane & 31;             // lanes 32..63 repeat lanes 0..31
    const bool wave0 = t < 64;

    // ---- forward: L y = b
    for (int kb = 0; kb < n; kb += NBS) {
        const int w = min(NBS, n - kb);
        if (wave0) {
            // y_j = x_j / L(j, j), then x_i -= L(i, j) y_j for the rows below j
            for (int j = 0; j < w; ++j) {
                if (li == j && lane < 32) {
                    const Rt d = re(lval<T, UPPER>(Ab, lda, kb + j, kb + j));
                    for (int r = 0; r < RC; ++r) X[(kb + j) * RC + r] = scale(X[(kb + j) * RC + r], Rt(1) / d);
                }
                wave_lds_sync();
                if (li > j && li < w && lane < 32) {
                    const T l = lval<T, UPPER>(Ab, lda, kb + li, kb + j);
                    for (int r = 0; r < RC; ++r) sub_mul(X[(kb + li) * RC + r], l, X[(kb + j) * RC + r]);
                }
                wave_lds_sync();
            }
        }
        __syncthreads();
        // rows below the block: x_k -= sum_j L(k, kb + j) y_{kb + j}
        for (int k = kb + w + t; k < n; k += THREADS) {
            T acc[RC];
            for (int r = 0; r < RC; ++r) acc[r] = X[k * RC + r];
            for (int j = 0; j < w; ++j) {
                const T l = lval<T, UPPER>(Ab, lda, k, kb + j);
                for (int r = 0; r < RC; ++r) sub_mul(acc[r], l, X[(kb + j) * RC + r]);
            }
            for (int r = 0; r < RC; ++r) X[k * RC + r] = acc[r];
        }
        __syncthreads();
    }

    // ---- backward: L^H x = y
    for (int kb = ((n - 1) / NBS) * NBS; kb >= 0; kb -= NBS) {
        const int w = min(NBS, n - kb);
        if (wave0) {
            // x_j = y_j / L(j, j), then x_i -= conj(L(j, i)) x_j for the rows above j
            for (int j = w - 1; j >= 0; --j) {
                if (li == j && lane < 32) {
                    const Rt d = re(lval<T, UPPER>(Ab, lda, kb + j, kb + j));
                    for (int r = 0; r < RC; ++r) X[(kb + j) * RC + r] = scale(X[(kb + j) * RC + r], Rt(1) / d);
                }
                wave_lds_sync();
                if (li < j && lane < 32) {
                    const T l = lval<T, UPPER>(Ab, lda, kb + j, kb + li);
                    for (int r = 0; r < RC; ++r) sub_conj_mul(X[(kb + li) * RC + r], l, X[(kb + j) * RC + r]);
                }
                wave_lds_sync();
            }
        }
        __syncthreads();
        // rows above the block: x_k -= sum_j conj(L(kb + j, k)) x_{kb + j}
        for (int k = t; k < kb; k += THREADS) {
            T acc[RC];
            for (int r = 0; r < RC; ++r) acc[r] = X[k * RC + r];
            for (int j = 0; j < w; ++j) {
                const T l = lval<T, UPPER>(Ab, lda, kb + j, k);
                for (int r = 0; r < RC; ++r) sub_conj_mul(acc[r], l, X[(kb + j) * RC + r]);
            }
            for (int r = 0; r < RC; ++r) X[k * RC + r] = acc[r];
        }
        __syncthreads();
    }

    for (int idx = t; idx < n * RC; idx += THREADS) {
        const int i = idx % n, r = idx / n;
        if (r < nr) Bb[int64_t(r0 + r) * ldb + i] = X[i * RC + r];
    }
}

// (the grid's second dimension covers the right-hand sides in blocks of RC)
constexpr int kMaxRhs = 65535 * RC;

template <typename T>
bool supported_t(int n, int nrhs) {
    return n >= 1 && n <= MAXN && nrhs >= 1 && nrhs <= kMaxRhs;
}

template <typename T>
hipError_t potrs_t(bool upper, int n, int nrhs, const void* A, int64_t lda, int64_t strideA,
                   void* B, int64_t ldb, int64_t strideB, int64_t batch, const int32_t* info,
                   hipStream_t s) {
    // one workgroup per item and block of RC right-hand sides; the grid's x
    // dimension covers the batch in slices of at most 2^31 - 1 items
    const int64_t ny = (nrhs + RC - 1) / RC;
    if (ny > 65535) return hipErrorInvalidValue;
    constexpr int64_t kMaxX = 0x7fffffff;
    hipError_t err = hipSuccess;
    for (int64_t b0 = 0; b0 < batch && err == hipSuccess; b0 += kMaxX) {
        const int64_t nb = batch - b0 < kMaxX ? batch - b0 : kMaxX;
        const T* a = static_cast<const T*>(A) + b0 * strideA;
        T* bb = static_cast<T*>(B) + b0 * strideB;
        const int32_t* inf = info != nullptr ? info + b0 : nullptr;
        const dim3 gd((unsigned)nb, (unsigned)ny), bd(THREADS);
        if (upper) err = launch(potrs_kernel<T, true>, gd, bd, 0, s, a, n, lda, strideA, bb, nrhs, ldb, strideB, nb, inf);
        else err = launch(potrs_kernel<T, false>, gd, bd, 0, s, a, n, lda, strideA, bb, nrhs, ldb, strideB, nb, inf);
    }
    return err;
}

}  // namespace potrs_detail
}  // namespace bl
