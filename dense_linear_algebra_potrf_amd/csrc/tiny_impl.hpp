// Tiny family (implementation header): batched Cholesky with each matrix held in registers.
//
// Prior art: the BatchLAS perf_potrf page, section "potrf: the tiny tier" (one
// matrix per lane partition, lane r owns row r, every value stays in
// registers) and section "The shared tiny-tier invariants" (no dynamic
// register indexing, failure writes as selects, every lane of a partition
// reaches every exchange, dead slots load the identity, Upper as a load/store
// transform).  That design targets 32-wide sub-groups; this one is built for
// 64-wide wavefronts:
//
//   * A matrix is owned by a partition of P lanes; lane q holds rows
//     q, q + P, ..., q + (R-1) P (R rows per lane), so a partition serves
//     orders n <= P R and a wavefront packs G = floor(64 / P) matrices.  P need
//     not be a power of two (n = 17 runs as 7 matrices of 9 lanes x 2 rows).
//   * Row block r only ever needs columns < (r + 1) P, so the triangular
//     shape of the work is kept: block 0 stops updating early.
//   * The pivot column is exchanged through LDS: each lane writes its entry of
//     column j once and every lane reads the column back with 16-byte
//     broadcast reads (the pages replaced per-element shuffles the same way,
//     section "The posv local-memory transpose").  The buffer is double
//     buffered by step parity, so no barrier is needed inside a wavefront.
//   * The rank-1 update uses the unscaled column: s_ik -= (s_ij / d) s_kj^H,
//     with d the updated (never stale) Schur pivot; the scaled factor column
//     l_ij = s_ij / sqrt(d) is written back afterwards.
//   * Failure handling follows the pages' info contract: d fails when
//     !(d > 0); the first failing column is kept and later updates stop
//     (section "potrf: correctness findings", item 6).
#pragma once

#include "families.hpp"

namespace bl {
namespace tiny_detail {

constexpr int kTinyWaves = 4;   // wavefronts per workgroup, each independent

// Dwords per partition row of the column buffer: >= nb * D, of the form
// 32 m + 4, so partitions of a wave start on different 16-byte bank groups.
constexpr int tiny_row_words(int nb, int d) {
    int w = (nb + 1) * d;   // one spare slot
    int m = (w - 4 + 31) / 32;
    if (m < 0) m = 0;
    return 32 * m + 4;
}

// Forward solve L y = b and backward solve L^H x = y for the rows a lane holds
// (the perf_potrf page, section "The fused posv tier", and section "posv: the
// backward solve costs a transpose").  The forward solve is column-oriented:
// once y_p is final its owner broadcasts it and every later row subtracts
// L(i, p) y_p.  The backward solve needs column p of L, which no lane holds;
// instead, at step p the owner of row p publishes that row through LDS and
// each lane reads the one entry L(p, i) it needs.  B is written only when the
// factorisation succeeded (info == 0), so a failed item leaves B unchanged.
template <typename T, int P, int R, int NRHS>
__device__ __forceinline__ void tiny_solves(const T (&a)[R][P * R], const typename Traits<T>::R (&invd)[R],
                                            uint32_t* ldsw, int parity_words, int roww, int p, int q,
                                            bool live, int n, int32_t inf, T* Bw, int nrhs,
                                            int64_t ldb, int64_t strideB)
{
    constexpr int NB = P * R;
    constexpr uint32_t S = sizeof(T);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bw);
    const uint32_t ldb_b = uint32_t(ldb) * S;
    uint32_t boff[R];
    static_for<0, R>([&](auto rr) {
        constexpr int r = rr;
        const int i = q + r * P;
        boff[r] = (live && i < n) ? uint32_t(p * strideB + i) * S : kBufOOB;
    });
    T y[R][NRHS];      // running right-hand sides
    T yf[R][NRHS];     // final y of the held rows
    static_for<0, R>([&](auto rr) {
        static_for<0, NRHS>([&](auto kk) {
            constexpr int r = rr, k = kk;
            const uint32_t off = (k < nrhs) ? boff[r] + uint32_t(k) * ldb_b : kBufOOB;
            y[r][k] = buf_load<T>(rb, off);
            yf[r][k] = zero<T>();
        });
    });
    // forward: L y = b, p ascending
    static_for<0, NB>([&](auto pp) {
        constexpr int pv = pp;
        constexpr int rp = pv / P;
        uint32_t* row = ldsw + (pv & 1) * parity_words + p * roww;
        const bool owner = q == pv % P;
        static_for<0, NRHS>([&](auto kk) {
            constexpr int k = kk;
            const T v = scale(y[rp][k], invd[rp]);
            yf[rp][k] = select(owner, v, yf[rp][k]);
            if (owner) lds_put<T>(row, NB + 1 + k, v);
        });
        wave_lds_sync();
        T yp[NRHS];
        static_for<0, NRHS>([&](auto kk) { yp[kk] = lds_get<T>(row, NB + 1 + kk); });
        static_for<rp, R>([&](auto rr) {
            constexpr int r = rr;
            static_for<0, NRHS>([&](auto kk) {
                constexpr int k = kk;
                sub_mul(y[r][k], a[r][pv], yp[k]);
            });
        });
    });
    // backward: L^H x = y, p descending
    T x[R][NRHS];
    static_for<0, R>([&](auto rr) {
        static_for<0, NRHS>([&](auto kk) { x[rr][kk] = yf[rr][kk]; });
    });
    T xf[R][NRHS];
    static_for<0, R>([&](auto rr) {
        static_for<0, NRHS>([&](auto kk) { xf[rr][kk] = zero<T>(); });
    });
    static_for_down<0, NB>([&](auto pp) {
        constexpr int pv = pp;
        constexpr int rp = pv / P;
        uint32_t* row = ldsw + (pv & 1) * parity_words + p * roww;
        const bool owner = q == pv % P;
        static_for<0, NRHS>([&](auto kk) {
            constexpr int k = kk;
            const T v = scale(x[rp][k], invd[rp]);
            xf[rp][k] = select(owner, v, xf[rp][k]);
            if (owner) lds_put<T>(row, NB + 1 + k, v);
        });
        if (owner) {
            static_for<0, pv>([&](auto cc) { lds_put<T>(row, cc, a[rp][cc]); });
        }
        wave_lds_sync();
        T xp[NRHS];
        static_for<0, NRHS>([&](auto kk) { xp[kk] = lds_get<T>(row, NB + 1 + kk); });
        // rows below p (i < p) take conj(L(p, i)) x_p; other rows only absorb junk
        static_for<0, cmin(R, rp + 1)>([&](auto rr) {
            constexpr int r = rr;
            const int i = q + r * P;
            const T lpi = lds_get<T>(row, i < pv ? i : NB);
            static_for<0, NRHS>([&](auto kk) {
                constexpr int k = kk;
                sub_conj_mul(x[r][k], lpi, xp[k]);
            });
        });
    });
    static_for<0, R>([&](auto rr) {
        static_for<0, NRHS>([&](auto kk) {
            constexpr int r = rr, k = kk;
            const uint32_t off = (inf == 0 && k < nrhs) ? boff[r] + uint32_t(k) * ldb_b : kBufOOB;
            buf_store<T>(rb, off, xf[r][k]);
        });
    });
}

// NRHS = 0: potrf.  NRHS > 0: posv for up to NRHS right-hand sides (nrhs at
// run time), with the factor kept in registers for both triangular solves.
template <typename T, int P, int R, bool UPPER, int NRHS>
__global__ __launch_bounds__(64 * kTinyWaves) void potrf_tiny_kernel(
    T* __restrict__ A, int n, int64_t lda, int64_t stride, int64_t batch,
    int32_t* __restrict__ info, T* __restrict__ B, int nrhs, int64_t ldb, int64_t strideB)
{
    using Rt = typename Traits<T>::R;
    constexpr int NB = P * R;
    constexpr int G = 64 / P;
    constexpr int PARTS = 63 / P + 1;     // includes a partial, dead tail partition
    constexpr int D = words<T>();
    constexpr int ROWW = tiny_row_words(NB + NRHS, D);
    __shared__ __attribute__((aligned(16))) uint32_t lds[kTinyWaves][2][PARTS][ROWW];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int p = lane / P;
    const int q = lane - p * P;
    const int64_t b_first = ((int64_t)blockIdx.x * kTinyWaves + wave) * G;   // wave-uniform
    const int64_t b = b_first + p;
    const bool live = (p < G) && (b < batch);
    // One buffer descriptor per wavefront; the host guarantees every byte offset
    // inside the wave's G matrices is below 2^31.  Masked elements use an
    // out-of-range offset, so they are neither read nor written.
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(A + b_first * stride);
    constexpr uint32_t S = sizeof(T);
    const uint32_t lda_b = uint32_t(lda) * S;
    uint32_t roff[R];
    static_for<0, R>([&](auto rr) {
        constexpr int r = rr;
        const int i = q + r * P;
        const uint32_t base = UPPER ? uint32_t(p * stride + int64_t(i) * lda) * S
                                    : uint32_t(p * stride + i) * S;
        roff[r] = (live && i < n) ? base : kBufOOB;
    });
    auto elem_off = [&](int r, int c) -> uint32_t {
        return UPPER ? roff[r] + uint32_t(c) * S : roff[r] + uint32_t(c) * lda_b;
    };

    // S(i, c) for c <= i: A(i, c) for Lower, conj(A(c, i)) for Upper.  Rows at
    // or beyond n, and dead partitions, hold the identity.
    T a[R][NB];
    static_for<0, R>([&](auto rr) {
        constexpr int r = rr;
        const int i = q + r * P;
        static_for<0, cmin(NB, (r + 1) * P)>([&](auto cc) {
            constexpr int c = cc;
            uint32_t off = elem_off(r, c);
            if constexpr (c >= r * P) off = (c <= i) ? off : kBufOOB;   // diagonal block
            T v = buf_load<T>(rsrc, off);
            if constexpr (UPPER) v = conj(v);
            if constexpr (c >= r * P) v = select(c == i && roff[r] == kBufOOB, one<T>(), v);
            a[r][c] = v;
        });
    });

    // Register slots a[r][k] with k > i (the row's upper part) are scratch: they
    // absorb updates but never feed a referenced slot, so a step needs no
    // per-row guards.  Rows at or beyond n hold the identity, so every one of
    // the NB steps can run unconditionally: a padding step sees d = 1 and
    // leaves the referenced part alone.  After a failed pivot the recurrence
    // continues (NaN from the failing column on); the leading columns are final
    // by then and info keeps the first failing column.
    //
    // Look-ahead: within step j, column j+1 is updated first and published to
    // LDS, and its 16-byte broadcast reads are issued before the rest of step
    // j's updates, so the exchange latency hides behind that arithmetic.
    // Column j is published at slots relative to j (row i -> slot i - j), so
    // the entries a step needs always start at slot 0: 16-byte aligned reads,
    // fewer of them as j grows.  Rows above j write to a spare slot at NB.
    auto publish = [&](auto jc) {
        constexpr int j = decltype(jc)::value;
        constexpr int rj = j / P;
        uint32_t* row = &lds[wave][j & 1][p][0];
        static_for<rj, R>([&](auto rr) {
            constexpr int r = rr;
            const int i = q + r * P;
            const int slot = (r == rj) ? ((i >= j) ? i - j : NB) : i - j;
            lds_put<T>(row, slot, a[r][j]);
        });
    };
    auto fetch = [&](auto jc, uint32_t (&w)[ROWW]) {
        constexpr int j = decltype(jc)::value;
        const uint4* row4 = reinterpret_cast<const uint4*>(
            __builtin_assume_aligned(&lds[wave][j & 1][p][0], 16));
        static_for<0, cdiv((NB - j) * D, 4)>([&](auto vv) {
            constexpr int v = vv;
            const uint4 x = row4[v];
            w[4 * v + 0] = x.x;
            w[4 * v + 1] = x.y;
            w[4 * v + 2] = x.z;
            w[4 * v + 3] = x.w;
        });
    };
    // entry for row k of column j (k >= j) in a fetched column
    auto colv = [&](const uint32_t (&w)[ROWW], int j, int k) -> T {
        return from_words<T>(&w[(k - j) * D]);
    };

    int32_t inf = 0;
    Rt invd[R];                 // 1 / L(i, i) of each held row (used by the solves)
    static_for<0, R>([&](auto rr) { invd[rr] = Rt(1); });
    uint32_t wcur[ROWW];
    publish(ic<0>{});
    wave_lds_sync();
    fetch(ic<0>{}, wcur);
    static_for<0, NB>([&](auto jj) {
        constexpr int j = jj;
        constexpr int rj = j / P;
        const Rt d = re(colv(wcur, j, j));
        inf = (inf == 0 && !(d > Rt(0))) ? (j + 1) : inf;
        const Rt inv = pivot_rcp(d);
        const Rt rs = pivot_rsq(d);
        T t[R];
        static_for<rj, R>([&](auto rr) {
            constexpr int r = rr;
            t[r] = scale(a[r][j], inv);
        });
        uint32_t wnext[ROWW];
        if constexpr (j + 1 < NB) {
            constexpr int rn = (j + 1) / P;
            static_for<rn, R>([&](auto rr) {
                constexpr int r = rr;
                sub_mul_conj(a[r][j + 1], t[r], colv(wcur, j, j + 1));
            });
            publish(ic<j + 1>{});
            wave_lds_sync();
            fetch(ic<j + 1>{}, wnext);
        }
        static_for<rj, R>([&](auto rr) {
            constexpr int r = rr;
            constexpr int kend = cmin(NB, (r + 1) * P);
            static_for<j + 2, kend>([&](auto kk) {
                constexpr int k = kk;
                sub_mul_conj(a[r][k], t[r], colv(wcur, j, k));
            });
            if constexpr (r == rj) {
                // the one row block that holds row j itself
                const bool diag = (q + r * P) == j;
                a[r][j] = select(diag, diag_value<T>(pivot_sqrt(d), UPPER), scale(a[r][j], rs));
                if constexpr (NRHS > 0) invd[r] = diag ? rs : invd[r];
            } else {
                a[r][j] = scale(a[r][j], rs);
            }
        });
        if constexpr (j + 1 < NB) {
            static_for<0, 4 * cdiv((NB - j - 1) * D, 4)>([&](auto kk) {
                constexpr int k = kk;
                wcur[k] = wnext[k];
            });
        }
    });

    if constexpr (NRHS > 0)
        tiny_solves<T, P, R, NRHS>(a, invd, &lds[wave][0][0][0], PARTS * ROWW, ROWW, p, q, live, n,
                                   inf, B + b_first * strideB, nrhs, ldb, strideB);

    static_for<0, R>([&](auto rr) {
        constexpr int r = rr;
        const int i = q + r * P;
        static_for<0, cmin(NB, (r + 1) * P)>([&](auto cc) {
            constexpr int c = cc;
            uint32_t off = elem_off(r, c);
            if constexpr (c >= r * P) off = (c <= i) ? off : kBufOOB;
            if constexpr (UPPER) buf_store<T>(rsrc, off, conj(a[r][c]));
            else buf_store<T>(rsrc, off, a[r][c]);
        });
    });
    if (live && q == 0 && info != nullptr) info[b] = inf;
}

// ---------------------------------------------------------------- configurations
template <int P_, int R_> struct TC {
    static constexpr int P = P_, R = R_, NB = P_ * R_;
};
template <typename... Cs> struct TList {};

// Ordered by order served (NB); the first entry with NB >= n is used.
template <typename T> struct TinyConfigs;
template <> struct TinyConfigs<float> {
    using type = TList<TC<4, 1>, TC<8, 1>, TC<6, 2>, TC<8, 2>, TC<9, 2>, TC<8, 3>, TC<8, 4>,
                       TC<11, 3>>;
};
template <> struct TinyConfigs<double> {
    using type = TList<TC<4, 1>, TC<8, 1>, TC<6, 2>, TC<8, 2>, TC<8, 3>, TC<8, 4>>;
};
template <> struct TinyConfigs<cfloat> {
    using type = TList<TC<4, 1>, TC<8, 1>, TC<6, 2>, TC<8, 2>, TC<8, 3>, TC<8, 4>>;
};
template <> struct TinyConfigs<cdouble> {
    using type = TList<TC<4, 1>, TC<8, 1>, TC<6, 2>, TC<8, 2>>;
};

// posv keeps more per lane (both solves' right-hand sides): smaller windows for
// the double types so that nothing spills.
template <typename T> struct PosvConfigs { using type = typename TinyConfigs<T>::type; };
template <> struct PosvConfigs<double> {
    using type = TList<TC<4, 1>, TC<8, 1>, TC<6, 2>, TC<8, 2>, TC<8, 3>>;
};
template <> struct PosvConfigs<cdouble> {
    using type = TList<TC<4, 1>, TC<8, 1>, TC<6, 2>, TC<8, 2>>;
};

template <typename F, typename C, typename... Cs>
bool pick_config(TList<C, Cs...>, int n, F&& f) {
    if (n <= C::NB) {
        f(C{});
        return true;
    }
    if constexpr (sizeof...(Cs) > 0) return pick_config(TList<Cs...>{}, n, f);
    else return false;
}

template <typename C, typename... Cs>
constexpr int last_nb(TList<C, Cs...>) {
    if constexpr (sizeof...(Cs) > 0) return last_nb(TList<Cs...>{});
    else return C::NB;
}

// The wave's G matrices must lie within 2^31 bytes of the wave's base, so the
// 32-bit buffer offsets (and the out-of-range mask) are exact.
template <typename T>
bool layout_ok_t(int n, int64_t stride) {
    bool ok = false;
    pick_config(typename TinyConfigs<T>::type{}, n, [&](auto c) {
        using C = decltype(c);
        constexpr int64_t G = 64 / C::P;
        ok = stride <= (int64_t(0x7fffffff) / int64_t(sizeof(T))) / G;
    });
    return ok;
}

template <typename T, typename List = typename TinyConfigs<T>::type>
bool geometry_t(int n, int64_t batch, Geometry& g) {
    return pick_config(List{}, n, [&](auto c) {
        using C = decltype(c);
        constexpr int G = 64 / C::P;
        constexpr int D = words<T>();
        g.family = FAM_TINY;
        g.P = C::P;
        g.R = C::R;
        g.G = G;
        g.threads = 64 * kTinyWaves;
        g.panel = 0;
        g.grid = (batch + G * kTinyWaves - 1) / (G * kTinyWaves);
        g.lds = int64_t(kTinyWaves) * 2 * (63 / C::P + 1) * tiny_row_words(C::NB, D) * 4;
    });
}

template <typename T>
hipError_t potrf_t(bool upper, int n, void* A, int64_t lda, int64_t stride, int64_t batch,
                   int32_t* info, hipStream_t s) {
    hipError_t err = hipErrorInvalidValue;
    pick_config(typename TinyConfigs<T>::type{}, n, [&](auto c) {
        using C = decltype(c);
        constexpr int G = 64 / C::P;
        const int64_t grid = (batch + G * kTinyWaves - 1) / (G * kTinyWaves);
        const dim3 gd((unsigned)grid), bd(64 * kTinyWaves);
        T* a = static_cast<T*>(A);
        T* nob = nullptr;
        if (upper)
            err = launch(potrf_tiny_kernel<T, C::P, C::R, true, 0>, gd, bd, 0, s, a, n, lda, stride,
                         batch, info, nob, 0, int64_t(0), int64_t(0));
        else
            err = launch(potrf_tiny_kernel<T, C::P, C::R, false, 0>, gd, bd, 0, s, a, n, lda, stride,
                         batch, info, nob, 0, int64_t(0), int64_t(0));
    });
    return err;
}

// posv: right-hand-side buckets NRHS = 1 and 4 (nrhs 2..4 run in the 4 bucket)
constexpr int kPosvMaxRhs = 4;

template <typename T>
bool posv_layout_ok_t(int n, int64_t strideA, int64_t strideB) {
    bool ok = false;
    pick_config(typename PosvConfigs<T>::type{}, n, [&](auto c) {
        using C = decltype(c);
        constexpr int64_t G = 64 / C::P;
        const int64_t lim = (int64_t(0x7fffffff) / int64_t(sizeof(T))) / G;
        ok = strideA <= lim && strideB <= lim;
    });
    return ok;
}

template <typename T>
hipError_t posv_t(bool upper, int n, int nrhs, void* A, int64_t lda, int64_t strideA, void* B,
                  int64_t ldb, int64_t strideB, int64_t batch, int32_t* info, hipStream_t s) {
    hipError_t err = hipErrorInvalidValue;
    pick_config(typename PosvConfigs<T>::type{}, n, [&](auto c) {
        using C = decltype(c);
        constexpr int G = 64 / C::P;
        const int64_t grid = (batch + G * kTinyWaves - 1) / (G * kTinyWaves);
        const dim3 gd((unsigned)grid), bd(64 * kTinyWaves);
        T* a = static_cast<T*>(A);
        T* bb = static_cast<T*>(B);
        auto go = [&](auto kern) {
            err = launch(kern, gd, bd, 0, s, a, n, lda, strideA, batch, info, bb, nrhs, ldb, strideB);
        };
        if (nrhs == 1) {
            if (upper) go(potrf_tiny_kernel<T, C::P, C::R, true, 1>);
            else go(potrf_tiny_kernel<T, C::P, C::R, false, 1>);
        } else {
            if (upper) go(potrf_tiny_kernel<T, C::P, C::R, true, kPosvMaxRhs>);
            else go(potrf_tiny_kernel<T, C::P, C::R, false, kPosvMaxRhs>);
        }
    });
    return err;
}

}  // namespace tiny_detail
}  // namespace bl
