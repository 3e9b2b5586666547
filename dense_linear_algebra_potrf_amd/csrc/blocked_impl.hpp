// Blocked family (implementation header): one workgroup factors one matrix of
// order up to 512, panel by panel, with the dense contraction on MFMA.
//
// Prior art: the BatchLAS perf_potrf page, sections on the blocked potrf (a
// panel factorisation, a triangular solve of the panel below its diagonal
// block, and a symmetric rank-k update that carries most of the flops).  The
// pages run these as separate batched launches per panel; on CDNA4 one
// workgroup keeps a whole matrix and runs the panels itself, left-looking, so
// the trailing data never makes a round trip through HBM between launches:
//
//   for each panel of NBP = 32 columns starting at k:
//     (i)   GEMM: P = S(k:n, k:k+32) - L(k:n, 0:k) L(k:k+32, 0:k)^T on MFMA
//           (v_mfma_*_16x16x4), each of 8 waves owning every eighth 16-row block;
//           P is kept in LDS (up to 512 x 33 elements), so the accumulators
//           are dead while the diagonal block is factored;
//     (ii)  the 32 x 32 diagonal block of P is factored on one wave, and the
//           inverse of its factor is built in the same sweep (every
//           elimination step is also applied to the columns of the identity),
//           info merged as k + j + 1;
//     (iii) the rows below are solved by a second MFMA product
//           L21 = P21 W^T with W = L11^-1 (lower triangular, zero blocks
//           skipped), both operands read from LDS;
//     then the panel is written to the matrix, where the next panels read it.
//
// S = A for Lower, S(i, c) = conj(A(c, i)) for Upper; for the real types the
// Upper form only swaps the address of each element.  Only the referenced
// triangle is read or written; rows beyond n load as zero and are never
// stored.  Failure handling follows the pages' info contract: the first
// failing pivot column is kept; later work runs on with NaN.
#pragma once

#include "families.hpp"

namespace bl {
namespace blocked_detail {

constexpr int NBP = 32;          // panel width
constexpr int WAVES = 8;         // wavefronts per workgroup
constexpr int MAXN = 512;        // largest order served
constexpr int MAXT = MAXN / 16 / WAVES;   // 16-row blocks per wave
constexpr int LDD = NBP + 1;     // padded row length of the LDS blocks

template <typename R> struct Mfma;
template <> struct Mfma<double> {
    typedef double v4 __attribute__((ext_vector_type(4)));
    static __device__ __forceinline__ v4 mac(double a, double b, v4 c) {
        return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
    }
    // Row of the 16 x 16 result held by register r of a lane in group g = lane / 16.
    static __device__ __forceinline__ constexpr int row(int r, int g) { return 4 * r + g; }
};
template <> struct Mfma<float> {
    typedef float v4 __attribute__((ext_vector_type(4)));
    static __device__ __forceinline__ v4 mac(float a, float b, v4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ constexpr int row(int r, int g) { return 4 * g + r; }
};

// The diagonal block of a panel, factored and inverted by one wavefront.
// Lanes 0..31 hold row i of the block (read from the panel in LDS); lanes
// 32..63 hold row i of the inverse being built, which starts as the identity.
// At step j the factor half publishes the pivot column and the inverse half's
// row j is published unscaled; rows below j take the Schur update of their
// entries right of column j, and the same elimination (multiplier S(i, j) / d_j)
// is applied to the inverse rows (entries up to column j, the rest are zero).
// Then column j of the factor is scaled by 1/sqrt(d_j) (diagonal sqrt(d_j)) and
// row j of the inverse likewise.  The block rows end as the factor L11, the
// inverse rows as W = L11^-1.  Rows at or beyond n are the identity.  The
// factor goes to the matrix, W to wm (row-major, zero above the diagonal) and
// the merged info to s_inf.  Plain unrolled loops keep v in registers.
template <typename R, bool UPPER>
__device__ __forceinline__ void factor_invert(const R* pb, R* wm, R* colx, int lane, int k,
                                              int n, int w, __amdgpu_buffer_rsrc_t rs,
                                              uint32_t ld, int32_t& s_inf)
{
    constexpr uint32_t S = sizeof(R);
    const int i = lane & 31;
    const bool inv_half = lane >= 32;
    const bool pad = k + i >= n;
    R* erow = colx + 2 * NBP;             // inverse-row exchange, 2 x NBP
    R v[NBP];
#pragma unroll
    for (int c = 0; c < NBP; ++c) {
        const R x = pb[i * LDD + c];
        const R id = (c == i) ? R(1) : R(0);
        v[c] = (inv_half || pad) ? id : x;
    }
    int32_t inf = s_inf;
#pragma unroll
    for (int j = 0; j < NBP; ++j) {
        const int par = j & 1;
        if (!inv_half) colx[par * NBP + i] = v[j];
        if (inv_half && i == j) {
#pragma unroll
            for (int c = 0; c <= j; ++c) erow[par * NBP + c] = v[c];
        }
        wave_lds_sync();
        const R d = colx[par * NBP + j];
        if (j < w) inf = (inf == 0 && !(d > R(0))) ? (k + j + 1) : inf;
        const R invd = pivot_rcp(d);
        const R rsd = pivot_rsq(d);
        R alpha = inv_half ? R(0) : v[j] * invd;
        alpha = __shfl(alpha, i);      // the factor half's multiplier for row i
        if (i > j) {
            // in groups of 8 columns, so that few LDS values are in flight at once
            if (!inv_half) {
#pragma unroll
                for (int c = j + 1; c < NBP; ++c) {
                    v[c] = fmadd(-alpha, colx[par * NBP + c], v[c]);
                    if ((c & 7) == 7) __builtin_amdgcn_sched_barrier(0);
                }
            } else {
#pragma unroll
                for (int c = 0; c <= j; ++c) {
                    v[c] = fmadd(-alpha, erow[par * NBP + c], v[c]);
                    if ((c & 7) == 7) __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        if (!inv_half) {
            v[j] = (i == j) ? pivot_sqrt(d) : (i > j ? v[j] * rsd : v[j]);
        } else if (i == j) {
#pragma unroll
            for (int c = 0; c <= j; ++c) v[c] = v[c] * rsd;
        }
    }
    if (!inv_half) {
        // the factor of the diagonal block goes straight to the matrix
#pragma unroll
        for (int c = 0; c < NBP; ++c) {
            const bool st = c <= i && c < w && !pad;
            const uint32_t o = UPPER ? (uint32_t(k + i) * ld + uint32_t(k + c)) * S
                                     : (uint32_t(k + c) * ld + uint32_t(k + i)) * S;
            buf_store<R>(rs, st ? o : kBufOOB, v[c]);
        }
    } else {
#pragma unroll
        for (int c = 0; c < NBP; ++c) wm[i * LDD + c] = v[c];
    }
    if (lane == 0) s_inf = inf;
}

template <typename R, bool UPPER>
__global__ __launch_bounds__(64 * WAVES) void potrf_blocked_kernel(
    R* __restrict__ A, int n, int64_t lda, int64_t stride, int64_t batch,
    int32_t* __restrict__ info)
{
    using M = Mfma<R>;
    using v4 = typename M::v4;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    R* pb = reinterpret_cast<R*>(smem);       // the panel P, MAXN rows x LDD
    R* wm = pb + MAXN * LDD;                  // inverse of the diagonal block's factor
    R* colx = wm + NBP * LDD;                 // pivot column exchange, 2 x 2 NBP
    int32_t* s_inf = reinterpret_cast<int32_t*>(colx + 4 * NBP);

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    constexpr uint32_t S = sizeof(R);
    const uint32_t ld = uint32_t(lda);
    // byte offset of S(row, col) inside the matrix (the host guarantees < 2^31)
    auto off = [&](int row, int col) -> uint32_t {
        return UPPER ? (uint32_t(row) * ld + uint32_t(col)) * S : (uint32_t(col) * ld + uint32_t(row)) * S;
    };

    for (int64_t b = blockIdx.x; b < batch; b += gridDim.x) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(A + b * stride);
        if (threadIdx.x == 0) *s_inf = 0;

        for (int k = 0; k < n; k += NBP) {
            // The lane index is re-read each panel and hidden from the
            // optimiser, so addresses derived from it are recomputed per panel
            // instead of being hoisted out of the loop, where they would stay
            // live (in registers) across the diagonal-block factorisation.
            int lane = threadIdx.x & 63;
            asm volatile("" : "+v"(lane));
            const int l16 = lane & 15, g = lane >> 4;
            const int w = min(NBP, n - k);            // panel width
            const int RB = (n - k + 15) >> 4;         // 16-row blocks of the panel
            {
                // ---- (i) accumulators start from S(k:n, k:k+w) (referenced part only)
                v4 acc[MAXT][2];
                static_for<0, MAXT>([&](auto tt) {
                    constexpr int t = tt;
                    const int ib = wave + WAVES * t;
                    static_for<0, 2>([&](auto cc) {
                        constexpr int cb = cc;
                        static_for<0, 4>([&](auto rr) {
                            constexpr int r = rr;
                            const int c = cb * 16 + M::row(r, g);
                            const int i = ib * 16 + l16;
                            const bool ref = ib < RB && k + i < n && c < w && i >= c;
                            acc[t][cb][r] = buf_load<R>(rs, ref ? off(k + i, k + c) : kBufOOB);
                        });
                    });
                });
                // GEMM over the factored columns q < k, four at a time.  Operands
                // live in two register sets (compile-time indices, so they stay
                // in registers); the loads of one step are in flight while the
                // MFMAs of the previous step run.  k is a multiple of 8 here.
                if (k > 0) {
                    const bool rowa0 = k + l16 < n, rowa1 = k + 16 + l16 < n;
                    R opa[2][2], opb[2][MAXT];
                    auto load_ops = [&](int q, auto setc) __attribute__((always_inline)) {
                        constexpr int st = decltype(setc)::value;
                        opa[st][0] = -buf_load<R>(rs, rowa0 ? off(k + l16, q + g) : kBufOOB);
                        opa[st][1] = -buf_load<R>(rs, rowa1 ? off(k + 16 + l16, q + g) : kBufOOB);
                        static_for<0, MAXT>([&](auto tt) {
                            constexpr int t = tt;
                            const int row = k + (wave + WAVES * t) * 16 + l16;
                            opb[st][t] = (wave + WAVES * t < RB)
                                             ? buf_load<R>(rs, row < n ? off(row, q + g) : kBufOOB)
                                             : R(0);
                        });
                    };
                    auto step = [&](auto setc) __attribute__((always_inline)) {
                        constexpr int st = decltype(setc)::value;
                        static_for<0, MAXT>([&](auto tt) {
                            constexpr int t = tt;
                            if (wave + WAVES * t < RB) {
                                acc[t][0] = M::mac(opa[st][0], opb[st][t], acc[t][0]);
                                acc[t][1] = M::mac(opa[st][1], opb[st][t], acc[t][1]);
                            }
                        });
                    };
                    load_ops(0, ic<0>{});
                    for (int q = 0; q < k; q += 8) {
                        load_ops(q + 4, ic<1>{});
                        step(ic<0>{});
                        if (q + 8 < k) load_ops(q + 8, ic<0>{});
                        step(ic<1>{});
                    }
                }
                // the panel P goes to LDS, row i of the panel at pb[i * LDD]
                static_for<0, MAXT>([&](auto tt) {
                    constexpr int t = tt;
                    const int ib = wave + WAVES * t;
                    if (ib < RB) {
                        static_for<0, 2>([&](auto cc) {
                            constexpr int cb = cc;
                            static_for<0, 4>([&](auto rr) {
                                constexpr int r = rr;
                                pb[(ib * 16 + l16) * LDD + cb * 16 + M::row(r, g)] = acc[t][cb][r];
                            });
                        });
                    }
                });
            }
            __syncthreads();

            // ---- (ii) factor and invert the diagonal block on wave 0
            if (wave == 0) factor_invert<R, UPPER>(pb, wm, colx, lane, k, n, w, rs, ld, *s_inf);
            __syncthreads();

            // ---- (iii) rows below the diagonal block: L21 = P21 W^T on MFMA,
            // with P21 (rows) and W^T (columns) read from LDS
            static_for<0, MAXT>([&](auto tt) {
                constexpr int t = tt;
                const int ib = wave + WAVES * t;
                if (ib >= 2 && ib < RB) {
                    static_for<0, 2>([&](auto pp) {
                        constexpr int cbp = pp;
                        v4 x = {R(0), R(0), R(0), R(0)};
                        static_for<0, 4 * (cbp + 1)>([&](auto uu) {   // W is lower triangular
                            constexpr int u = uu;
                            const int c = 4 * u + g;                  // contraction index
                            const R ao = pb[(ib * 16 + l16) * LDD + c];
                            const R bo = wm[(cbp * 16 + l16) * LDD + c];
                            x = M::mac(ao, bo, x);
                        });
                        static_for<0, 4>([&](auto rr) {
                            constexpr int r = rr;
                            const int row = k + ib * 16 + M::row(r, g);
                            const int col = cbp * 16 + l16;
                            const bool st = row < n && col < w;
                            buf_store<R>(rs, st ? off(row, k + col) : kBufOOB, x[r]);
                        });
                    });
                }
            });
            __syncthreads();   // the panel is in memory before the next GEMM reads it
        }
        if (threadIdx.x == 0 && info != nullptr) info[b] = *s_inf;
        __syncthreads();
    }
}

// ---------------------------------------------------------------- host side
constexpr int64_t kMaxGrid = int64_t(1) << 20;

template <typename R>
constexpr int64_t lds_bytes() {
    return int64_t(MAXN * LDD + NBP * LDD + 4 * NBP) * sizeof(R) + 16;
}

template <typename R>
bool supported_t(int n, int64_t lda) {
    return n >= 1 && n <= MAXN && lda * int64_t(n) * int64_t(sizeof(R)) < (int64_t(1) << 31);
}

template <typename R>
bool geometry_t(int n, int64_t batch, Geometry& g) {
    if (n < 1 || n > MAXN) return false;
    g.family = FAM_BLOCKED;
    g.P = g.R = g.G = 0;
    g.threads = 64 * WAVES;
    g.panel = NBP;
    g.grid = batch < kMaxGrid ? batch : kMaxGrid;
    g.lds = lds_bytes<R>();
    return true;
}

template <typename R>
hipError_t potrf_t(bool upper, int n, void* A, int64_t lda, int64_t stride, int64_t batch,
                   int32_t* info, hipStream_t s) {
    const dim3 gd((unsigned)(batch < kMaxGrid ? batch : kMaxGrid)), bd(64 * WAVES);
    R* a = static_cast<R*>(A);
    const size_t shm = size_t(lds_bytes<R>());
    if (upper) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(potrf_blocked_kernel<R, true>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(shm));
        if (e != hipSuccess) return e;
        return launch(potrf_blocked_kernel<R, true>, gd, bd, shm, s, a, n, lda, stride, batch, info);
    }
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(potrf_blocked_kernel<R, false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(shm));
    if (e != hipSuccess) return e;
    return launch(potrf_blocked_kernel<R, false>, gd, bd, shm, s, a, n, lda, stride, batch, info);
}

}  // namespace blocked_detail
}  // namespace bl
