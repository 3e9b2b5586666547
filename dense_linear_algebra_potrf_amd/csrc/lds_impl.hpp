// LDS family (implementation header): one workgroup factors one matrix.
//
// Prior art: the BatchLAS perf_potrf page, sections on the work-group tiers
// (the matrix is staged in shared local memory, a right-looking factorisation
// runs over it with barriers after staging, between reading the pivot and
// overwriting it, and at the end of a panel; register tiles carry the trailing
// update).  Built for CDNA4 as follows:
//
//   * Staging.  The referenced triangle is read from HBM with consecutive
//     threads on consecutive elements of a column (coalesced), and written to
//     an LDS image of S in row-major order with a padded row length NB + 1
//     (S = A for Lower, S(i, c) = conj(A(c, i)) for Upper, so both uplos run
//     the same Lower recurrence).  The store goes back the same way.  The
//     other triangle and the padding are neither read nor written.
//   * Register tiles.  The lower triangle of S is cut into TR x TC tiles, one
//     per thread, numbered column block by column block.  As the
//     factorisation advances, whole waves of finished column blocks stop
//     issuing work and leave their SIMD to other workgroups on the CU.
//   * One barrier per column.  At step j the owners of column j publish it
//     (unscaled) into a double-buffered column buffer; after the barrier every
//     thread reads the Schur pivot d = S(j, j), updates its tile with
//     S(i, k) -= S(i, j) conj(S(k, j)) / d for k > j, and the owners replace
//     column j by the factor column (S(i, j) / sqrt(d), diagonal sqrt(d)).
//     Updates of slots above the diagonal only touch scratch that is never
//     stored.
//   * info: the first j with !(d > 0) (zero, negative and NaN pivots fail),
//     never overwritten; the recurrence runs on, so the leading columns hold
//     the factor of the leading block.
#pragma once

#include "families.hpp"

namespace bl {
namespace lds_detail {

// Number of tiles of the lower triangle (tiles that hold at least one element
// on or below the diagonal) for an NB x NB matrix cut in TR x TC tiles.
constexpr int lower_tiles(int nb, int tr, int tc) {
    int cnt = 0;
    for (int cb = 0; cb < nb / tc; ++cb) cnt += nb / tr - (cb * tc) / tr;
    return cnt;
}
constexpr int round_up(int a, int b) { return (a + b - 1) / b * b; }

template <int NB_, int TR_, int TC_> struct LC {
    static constexpr int NB = NB_, TR = TR_, TC = TC_;
    static constexpr int TILES = lower_tiles(NB_, TR_, TC_);
    static constexpr int THREADS = round_up(TILES, 64);
    static_assert(NB_ % TR_ == 0 && NB_ % TC_ == 0, "tile shape");
    static_assert(THREADS <= 1024, "workgroup size");
};
template <typename... Cs> struct LList {};

template <typename T> struct LdsConfigs;
template <> struct LdsConfigs<float> {
    using type = LList<LC<48, 4, 2>, LC<64, 4, 2>, LC<96, 4, 2>>;
};
template <> struct LdsConfigs<double> {
    using type = LList<LC<48, 4, 2>, LC<64, 4, 2>, LC<96, 4, 2>>;
};
template <> struct LdsConfigs<cfloat> {
    using type = LList<LC<48, 4, 2>, LC<64, 4, 2>, LC<96, 4, 2>>;
};
template <> struct LdsConfigs<cdouble> {
    using type = LList<LC<48, 4, 2>, LC<64, 4, 2>>;
};

template <typename T, int NB>
constexpr int64_t lds_bytes() {
    return int64_t(NB) * (NB + 1) * sizeof(T) + 2 * int64_t(NB) * sizeof(T);
}

template <typename T, typename C, bool UPPER>
__global__ __launch_bounds__(C::THREADS) void potrf_lds_kernel(
    T* __restrict__ A, int n, int64_t lda, int64_t stride, int64_t batch,
    int32_t* __restrict__ info)
{
    using Rt = typename Traits<T>::R;
    constexpr int NB = C::NB, TR = C::TR, TC = C::TC, THREADS = C::THREADS;
    constexpr int LD = NB + 1;                      // padded row length of the image
    constexpr int LOADS = cdiv(NB * NB, THREADS);   // column-major positions per thread
    __shared__ T img[NB * LD];
    __shared__ T colbuf[2][NB];

    const int t = threadIdx.x;

    // ---- this thread's tile: column block cb, row block rb (column-block-major order)
    int rb = 0, cb = 0;
    bool valid = false;
    {
        int idx = t;
        for (int c = 0; c < NB / TC; ++c) {
            const int first = (c * TC) / TR;
            const int cnt = NB / TR - first;
            if (!valid && idx < cnt) {
                rb = first + idx;
                cb = c;
                valid = true;
            }
            idx -= cnt;
        }
    }
    const int i0 = rb * TR, k0 = cb * TC;
    // first column-major position handled by this thread, and the per-pass step
    const int pi0 = t % n, pc0 = t / n;
    const int di = THREADS % n, dc = THREADS / n;

    for (int64_t b = blockIdx.x; b < batch; b += gridDim.x) {
        T* __restrict__ Ab = A + b * stride;

        // ---- stage the referenced triangle into the image (coalesced loads,
        // issued CH at a time so that several are in flight per thread)
        {
            constexpr int CH = 8;
            int i = pi0, c = pc0;
            static_for<0, cdiv(LOADS, CH)>([&](auto hh) {
                constexpr int h = hh;
                constexpr int cnt = cmin(CH, LOADS - h * CH);
                T v[CH];
                int ii[CH], cc[CH];
                static_for<0, cnt>([&](auto ss) {
                    constexpr int q = ss;
                    const bool ref = c < n && (UPPER ? i <= c : i >= c);
                    v[q] = ref ? Ab[int64_t(c) * lda + i] : zero<T>();
                    ii[q] = ref ? i : -1;
                    cc[q] = c;
                    i += di;
                    c += dc;
                    if (i >= n) { i -= n; c += 1; }
                });
                static_for<0, cnt>([&](auto ss) {
                    constexpr int q = ss;
                    if (ii[q] >= 0) {
                        if constexpr (UPPER) img[cc[q] * LD + ii[q]] = conj(v[q]);
                        else img[ii[q] * LD + cc[q]] = v[q];
                    }
                });
            });
        }
        __syncthreads();

        T s[TR][TC];
        static_for<0, TR>([&](auto rr) {
            static_for<0, TC>([&](auto cc) {
                s[rr][cc] = img[(i0 + rr) * LD + k0 + cc];
            });
        });

        // ---- right-looking factorisation, one column per step
        int32_t inf = 0;
        for (int j = 0; j < n; ++j) {
            const int par = j & 1;
            const bool owner = valid && cb == j / TC;
            const int jc = j - k0;   // column of j inside an owner's tile
            if (owner) {
                static_for<0, TR>([&](auto rr) {
                    constexpr int r = rr;
                    T v = s[r][0];
                    static_for<1, TC>([&](auto cc) { v = select(jc == cc, s[r][cc], v); });
                    if (i0 + r >= j) colbuf[par][i0 + r] = v;
                });
            }
            __syncthreads();
            const Rt d = re(colbuf[par][j]);
            inf = (inf == 0 && !(d > Rt(0))) ? (j + 1) : inf;
            if (valid && k0 + TC - 1 > j && i0 + TR - 1 > j) {
                const Rt inv = pivot_rcp(d);
                T ci[TR], wk[TC];
                static_for<0, TR>([&](auto rr) { ci[rr] = colbuf[par][i0 + rr]; });
                static_for<0, TC>([&](auto cc) { wk[cc] = scale(conj(colbuf[par][k0 + cc]), inv); });
                static_for<0, TC>([&](auto cc) {
                    constexpr int c = cc;
                    if (k0 + c > j) {
                        static_for<0, TR>([&](auto rr) { sub_mul(s[rr][c], ci[rr], wk[c]); });
                    }
                });
            }
            if (owner) {
                const Rt rs = pivot_rsq(d);
                const T dg = diag_value<T>(pivot_sqrt(d), UPPER);
                static_for<0, TR>([&](auto rr) {
                    constexpr int r = rr;
                    const int i = i0 + r;
                    static_for<0, TC>([&](auto cc) {
                        constexpr int c = cc;
                        const T fin = (i == j) ? dg : scale(s[r][c], rs);
                        s[r][c] = select(jc == c && i >= j, fin, s[r][c]);
                    });
                });
            }
        }

        // ---- write the factor back through the image (coalesced stores)
        static_for<0, TR>([&](auto rr) {
            static_for<0, TC>([&](auto cc) {
                if (valid) img[(i0 + rr) * LD + k0 + cc] = s[rr][cc];
            });
        });
        __syncthreads();
        {
            int i = pi0, c = pc0;
            static_for<0, LOADS>([&](auto ss) {
                const bool ref = c < n && (UPPER ? i <= c : i >= c);
                if (ref) {
                    if constexpr (UPPER) Ab[int64_t(c) * lda + i] = conj(img[c * LD + i]);
                    else Ab[int64_t(c) * lda + i] = img[i * LD + c];
                }
                i += di;
                c += dc;
                if (i >= n) { i -= n; c += 1; }
            });
        }
        if (t == 0 && info != nullptr) info[b] = inf;
        __syncthreads();   // the image and column buffer are reused by the next matrix
    }
}

// ---------------------------------------------------------------- host side
template <typename F, typename C, typename... Cs>
bool pick(LList<C, Cs...>, int n, F&& f) {
    if (n <= C::NB) {
        f(C{});
        return true;
    }
    if constexpr (sizeof...(Cs) > 0) return pick(LList<Cs...>{}, n, f);
    else return false;
}
template <typename C, typename... Cs>
constexpr int last_nb(LList<C, Cs...>) {
    if constexpr (sizeof...(Cs) > 0) return last_nb(LList<Cs...>{});
    else return C::NB;
}

// Workgroups per launch: one per matrix, capped; larger batches loop.
constexpr int64_t kMaxGrid = int64_t(1) << 20;

template <typename T>
bool geometry_t(int n, int64_t batch, Geometry& g) {
    return pick(typename LdsConfigs<T>::type{}, n, [&](auto c) {
        using C = decltype(c);
        g.family = FAM_LDS;
        g.P = g.R = g.G = 0;
        g.threads = C::THREADS;
        g.panel = C::TC;
        g.grid = batch < kMaxGrid ? batch : kMaxGrid;
        g.lds = lds_bytes<T, C::NB>();
    });
}

template <typename T>
hipError_t potrf_t(bool upper, int n, void* A, int64_t lda, int64_t stride, int64_t batch,
                   int32_t* info, hipStream_t s) {
    hipError_t err = hipErrorInvalidValue;
    pick(typename LdsConfigs<T>::type{}, n, [&](auto c) {
        using C = decltype(c);
        const dim3 gd((unsigned)(batch < kMaxGrid ? batch : kMaxGrid)), bd(C::THREADS);
        T* a = static_cast<T*>(A);
        if (upper)
            err = launch(potrf_lds_kernel<T, C, true>, gd, bd, 0, s, a, n, lda, stride, batch, info);
        else
            err = launch(potrf_lds_kernel<T, C, false>, gd, bd, 0, s, a, n, lda, stride, batch, info);
    });
    return err;
}

}  // namespace lds_detail
}  // namespace bl
