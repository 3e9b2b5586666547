// Blocked family (implementation header): one workgroup factors one matrix of
// order up to 512, panel by panel, with the dense contraction on MFMA.
//
// Prior art: the BatchLAS perf_potrf page, sections on the blocked potrf (a
// panel factorisation, a triangular solve of the panel below its diagonal
// block, and a symmetric rank-k update that carries most of the flops).  The
// pages run these as separate batched launches per panel; on CDNA4 one
// workgroup of four wavefronts runs the panels of one matrix itself,
// left-looking:
//
//   for each panel starting at column k:
//     (i)   GEMM: P = S(k:n, k:k+w) - L(k:n, 0:k) L(k:k+w, 0:k)^T on MFMA
//           (v_mfma_*_16x16x4, accumulated as L L^T - S so that no operand needs
//           negating): the diagonal block into LDS, the 32-row superblocks
//           below it in registers;
//     (ii)  one wave factors the diagonal block in 32 x 32 blocks and forms the
//           inverse W of each factor, info merged as k + j + 1, while the
//           other waves run their GEMMs;
//     (iii) the rows below are solved by a second MFMA product
//           L21 = P21 W^T (W lower triangular, zero blocks skipped) straight
//           from the GEMM's accumulators, and L21 is written over S, where
//           the next panels read it.
//   The real types take 64-column panels (the left-looking GEMM re-reads
//   the columns of L left of k once per panel, so the wider panel halves
//   that traffic; factor_matrix_wide), the complex types 32-column ones
//   (factor_matrix).  Only the diagonal blocks, their inverses and a few
//   vectors live in LDS, so two workgroups (matrices) share a compute unit:
//   while one factors a diagonal block on one wave, the other keeps the
//   matrix cores busy.
//
// S = A for Lower, S(i, c) = conj(A(c, i)) for Upper; for the real types the
// Upper form only swaps the address of each element.  The complex types
// split each complex product into four real MFMAs on separate real and
// imaginary accumulators (the pages' complex trailing update is a ConjTrans
// GEMM).  Only the referenced triangle is read or written; rows beyond n load
// as zero and are never stored.  Failure handling follows the pages' info
// contract: the first failing pivot column is kept; the columns before it are
// final, and the rest is not meaningful.
#pragma once

#include "families.hpp"

namespace bl {
namespace blocked_detail {

constexpr int NBP = 32;          // panel width
constexpr int WAVES = 4;         // wavefronts per workgroup
constexpr int LDD = NBP + 1;     // padded row length of the LDS blocks

// Largest order served (the loops are not bounded by it; it is the range the
// family is built and tested for).
template <typename T> struct Shape {
    static constexpr int MAXN = 512;
};
// The diagonal block is factored in double for the real types and in the
// element type itself for the complex ones.
template <typename T> struct FactorType {
    using type = typename std::conditional<Traits<T>::cplx, T, double>::type;
};
template <typename To, typename From> __device__ __forceinline__ To cvt(const From& x) {
    if constexpr (Traits<To>::cplx) return x;
    else return To(x);
}

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

// Complex multiply-accumulate on split planes: (cr, ci) += conj(a) b when CONJ,
// else a b, as four real MFMAs.
template <bool CONJ, typename R, typename V>
__device__ __forceinline__ void cmac(R ar, R ai, R br, R bi, V& cr, V& ci) {
    using M = Mfma<R>;
    const R nai = -ai;
    cr = M::mac(ar, br, cr);
    cr = M::mac(CONJ ? ai : nai, bi, cr);
    ci = M::mac(ar, bi, ci);
    ci = M::mac(CONJ ? nai : ai, br, ci);
}

// LDS pointers as 32-bit offsets (address space 3), and a read pointer whose
// value the optimiser cannot know before dep is computed (the reads through it
// stay after dep's computation).
template <typename V> using lds_cptr = __attribute__((address_space(3))) const V*;
template <typename V> __device__ __forceinline__ uint32_t lds_offset(const V* p) {
    return uint32_t(uintptr_t((lds_cptr<V>)p));   // (an address-space cast)
}
template <typename V, typename D> __device__ __forceinline__ lds_cptr<V> lds_after(uint32_t off, D dep) {
    asm volatile("" : "+v"(off) : "v"(dep));
    return (lds_cptr<V>)uintptr_t(off);
}

// A 32 x 32 diagonal block (real types), factored in double by one
// wavefront.  Lane i (i = lane mod 32; the upper half of the wave repeats the
// lower half) holds row i of the block.  At step j the pivot d = S(j, j) and
// S(j + 1, j) are read from lanes j and j + 1 directly (lane reads), rows
// below j take the Schur update of their entries right of column j with the
// multiplier S(i, j) / d, and column j is scaled by 1/sqrt(d) (the diagonal
// becomes sqrt(d)).  Column j + 1 is updated first and published to LDS, from
// where the other lanes read it in one batch at the next step, off the chain
// of dependent pivots.  Rows at or beyond n are the identity.  The factor goes
// to the matrix and back into the block buffer pb, 1/L(j, j) to rdiag, and the
// inverse W of the factor (below) to wm for the solves.  The LDS stores of the
// step loop are unconditional (the two halves of the wave write identical
// values): stores under a lane condition split the code into many small
// blocks, after which the compiler keeps hundreds of values live and spills.
template <typename T, bool UPPER>
__device__ __forceinline__ void factor_diag(T* pb, T* wm, double* colx, double* rdiag,
                                            int lane, int k, int n, int w,
                                            __amdgpu_buffer_rsrc_t rs, uint32_t ld, int32_t& s_inf)
{
    constexpr uint32_t S = sizeof(T);
    const int i = lane & 31;
    const bool writer = lane < 32;
    const bool pad = k + i >= n;
    double v[NBP];
    static_for<0, NBP>([&](auto cc) {
        constexpr int c = cc;
        // (the read is made opaque so that it stays unconditional: sunk into a
        // branch under the select, it splits the code into small blocks and
        // the kernel spills)
        double x = double(pb[i * LDD + c]);
        asm volatile("" : "+v"(x));
        v[c] = pad ? ((c == i) ? 1.0 : 0.0) : x;
    });
    int32_t inf = s_inf;
    double rsd_mine = 1.0;
    colx[i] = v[0];
    wave_lds_sync();
    const uint32_t cxo = lds_offset(colx);
    // a lane's value of x, read by the whole wave (two 32-bit lane reads)
    auto lane_read = [](double x, int src) __attribute__((always_inline)) {
        const uint64_t u = __builtin_bit_cast(uint64_t, x);
        const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(u), src);
        const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(u >> 32), src);
        return __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
    };
    static_for<0, NBP>([&](auto jj) {
        constexpr int j = jj;
        // The pivot S(j, j) and S(j + 1, j), which the next pivot's chain
        // needs, are read from lanes j and j + 1 directly; the rest of column
        // j (rows j + 2..), published at step j - 1, comes from LDS in one
        // batch (consumed one by one, the reads would each wait for the
        // previous one), off that chain.
        const double d = lane_read(v[j], j);
        double s1 = 0.0;
        if constexpr (j + 1 < NBP) s1 = lane_read(v[j], j + 1);
        double cv[NBP];
        if constexpr (j + 2 < NBP) {
            const lds_cptr<double> col = lds_after<double>(cxo + uint32_t((j & 1) * NBP) * 8u, v[j]);
            static_for<j + 2, NBP>([&](auto mm) { cv[mm] = col[mm]; });
        }
        __builtin_amdgcn_sched_barrier(0);
        if (j < w) inf = (inf == 0 && !(d > 0.0)) ? (k + j + 1) : inf;
        // the multiplier S(i, j) / d from the reciprocal of d, the shorter
        // dependent chain; sqrt(d) and 1/sqrt(d), for column j itself, run
        // beside it
        double sq, rsd;
        pivot_sqrt_rsq(d, sq, rsd);
        const double beta = v[j] * pivot_rcp(d);
        // rows at or above j only touch slots right of the diagonal (unused)
        if constexpr (j + 1 < NBP) {
            v[j + 1] = __builtin_fma(-beta, s1, v[j + 1]);
            colx[((j + 1) & 1) * NBP + i] = v[j + 1];
        }
        static_for<j + 2, NBP>([&](auto mm) {
            constexpr int m = mm;
            v[m] = __builtin_fma(-beta, cv[m], v[m]);
        });
        v[j] = (i == j) ? sq : v[j] * rsd;            // rows above j: unused slot
        rsd_mine = (i == j) ? rsd : rsd_mine;
        wave_lds_sync();
    });
    // the factor: to the matrix, and back into the block buffer
    static_for<0, NBP>([&](auto cc) {
        constexpr int c = cc;
        const bool st = writer && c <= i && c < w && !pad;
        const uint32_t o = UPPER ? (uint32_t(k + i) * ld + uint32_t(k + c)) * S
                                 : (uint32_t(k + c) * ld + uint32_t(k + i)) * S;
        buf_store<T>(rs, st ? o : kBufOOB, T(v[c]));
        pb[i * LDD + c] = (c <= i) ? T(v[c]) : T(0);
    });
    rdiag[i] = rsd_mine;
    wave_lds_sync();
    // Inverse W = L11^-1 in 16 x 16 blocks.  The diagonal blocks W11 and W22
    // (inverses of the diagonal blocks of L11) by forward substitution,
    //     W(m, c) = (delta(m, c) - sum_{p < m} L(m, p) W(p, c)) / L(m, m),
    // lane i forming column i mod 16 of block i / 16, both blocks at once (a
    // chain of 16 rows instead of 32); row m + 1 of the block is read in one
    // batch while row m is summed, the sum running as four interleaved
    // partial sums.  Then W21 = -W22 (L21 W11) as two 16 x 16 x 16 MFMA
    // products, the first one's result registers feeding the second as its B
    // operand (register r of lane group g holds row row(r, g) of L21 W11, four
    // distinct rows over the groups).  W12 = 0.
    {
        const int blk = i >> 4, ci = i & 15;
        const uint32_t pbo = lds_offset(pb) + uint32_t(16 * blk * (LDD + 1)) * uint32_t(sizeof(T));
        double x[16];
        double lr[2][16];   // row m in lr[m & 1], row m + 1 arriving in the other
        static_for<0, 16>([&](auto mm) {
            constexpr int m = mm;
            if constexpr (m + 1 < 16) {
                const lds_cptr<T> row = lds_after<T>(pbo + uint32_t((m + 1) * LDD) * uint32_t(sizeof(T)),
                                                     x[m > 0 ? m - 1 : 0]);
                static_for<0, m + 1>([&](auto pp) { lr[(m + 1) & 1][pp] = double(row[pp]); });
            }
            const double rd = rdiag[16 * blk + m];
            __builtin_amdgcn_sched_barrier(0);
            double acc[4] = {(m == ci) ? 1.0 : 0.0, 0.0, 0.0, 0.0};
            static_for<0, m>([&](auto pp) {
                constexpr int p = pp;
                acc[p & 3] = __builtin_fma(-lr[m & 1][p], x[p], acc[p & 3]);
            });
            x[m] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) * rd;
        });
        static_for<0, 16>([&](auto mm) {
            constexpr int m = mm;
            wm[(16 * blk + m) * LDD + 16 * blk + ci] = T(x[m]);
        });
        if (blk == 1) static_for<0, 16>([&](auto mm) { wm[mm * LDD + 16 + ci] = T(0); });   // W12

    }
    wave_lds_sync();
    {
        using MD = Mfma<double>;
        const int l16 = lane & 15, g = (lane >> 4) & 3;
        typename MD::v4 t = {0.0, 0.0, 0.0, 0.0}, y = {0.0, 0.0, 0.0, 0.0};
        static_for<0, 4>([&](auto uu) {        // t = L21 W11
            constexpr int u = uu;
            t = MD::mac(double(pb[(16 + l16) * LDD + 4 * u + g]), double(wm[(4 * u + g) * LDD + l16]), t);
        });
        static_for<0, 4>([&](auto rr) {        // y = W22 t
            constexpr int r = rr;
            const double tr = t[r];
            y = MD::mac(double(wm[(16 + l16) * LDD + 16 + MD::row(r, g)]), tr, y);
        });
        static_for<0, 4>([&](auto rr) {
            constexpr int r = rr;
            const double yr = y[r];
            wm[(16 + MD::row(r, g)) * LDD + l16] = T(-yr);
        });
    }
    if (lane == 0) s_inf = inf;
}

// Complex types: the same factorisation and inverse worked in place in LDS
// (row i of the block at pb[i * LDD], lane i owning row i, the inverse built
// column by column in wm), so that no lane holds a whole row: with the row and
// the column of the inverse in registers the complex kernels spill.  The
// column of step j is read by every lane before its owners rescale it (LDS
// instructions of one wave complete in order).
template <typename T, bool UPPER>
__device__ __forceinline__ void factor_invert_inplace(T* pb, T* wm, typename Traits<T>::R* rdiag,
                                                      int lane, int k, int n, int w,
                                                      __amdgpu_buffer_rsrc_t rs, uint32_t ld,
                                                      int32_t& s_inf)
{
    using R = typename Traits<T>::R;
    constexpr uint32_t S = sizeof(T);
    const int i = lane & 31;
    const bool writer = lane < 32;
    const bool pad = k + i >= n;
    T* row = pb + i * LDD;
#pragma unroll 1
    for (int c = 0; c < NBP; ++c) row[c] = select(pad, select(c == i, one<T>(), zero<T>()), row[c]);
    wave_lds_sync();
    int32_t inf = s_inf;
#pragma unroll 1
    for (int j = 0; j < NBP; ++j) {
        const R d = re(pb[j * LDD + j]);
        if (j < w) inf = (inf == 0 && !(d > R(0))) ? (k + j + 1) : inf;
        R sq, rsd;
        pivot_sqrt_rsq(d, sq, rsd);
        const T lij = row[j];
        const T beta = scale(lij, rsd * rsd);       // S(i, j) / d
        // rows at or above j only touch slots right of the diagonal (unused)
#pragma unroll 2
        for (int m = j + 1; m < NBP; ++m) {
            T v = row[m];
            sub_mul_conj(v, beta, pb[m * LDD + j]);
            row[m] = v;
        }
        wave_lds_sync();
        row[j] = select(i == j, diag_value<T>(sq, UPPER), select(i > j, scale(lij, rsd), lij));
        rdiag[j] = rsd;
        wave_lds_sync();
    }
#pragma unroll 1
    for (int c = 0; c < NBP; ++c) {
        const bool st = writer && c <= i && c < w && !pad;
        const uint32_t o = UPPER ? (uint32_t(k + i) * ld + uint32_t(k + c)) * S
                                 : (uint32_t(k + c) * ld + uint32_t(k + i)) * S;
        buf_store<T>(rs, st ? o : kBufOOB, UPPER ? conj(row[c]) : row[c]);
    }
    // column i of conj(W), W = L11^-1, by forward substitution
#pragma unroll 1
    for (int m = 0; m < NBP; ++m) {
        T acc = select(m == i, one<T>(), zero<T>());
#pragma unroll 2
        for (int p = 0; p < m; ++p) sub_mul(acc, pb[m * LDD + p], conj(wm[p * LDD + i]));
        wm[m * LDD + i] = conj(scale(acc, rdiag[m]));
    }
    if (lane == 0) s_inf = inf;
}

// The GEMM of one panel starting at column kp:
//     P = S(kp:n, kp:kp+w) - L(kp:n, 0:kp) L(kp:kp+w, 0:kp)^H,
// accumulated on MFMA as L L^H - S (so that no operand needs negating) and
// written, negated back, over S in the matrix, except the diagonal block,
// which goes to LDS for the factorisation (row i at p11[i * LDD]; columns at
// or beyond w as 0).  accumulate() adds the columns [q0, q1) of L.
//
// A wave owns the 32-row superblocks sb = sb0 + GW s (s < MAXS) of the panel,
// each split into its even and odd rows (two 16-row MFMA tiles); the panel's
// 32 columns are split the same way (cb = 0: even columns, cb = 1: odd
// columns), so that a lane loads two consecutive rows of a column at once
// where the layout allows it.  MFMA roles: the A operand runs over the panel's
// columns c (rows kp + c of L), the B operand over the panel's rows i; the
// result is P^T tile by tile.  With PAIRED (fp64 Lower, n even), a lane loads
// rows 2 l16 and 2 l16 + 1 of one column with a single 16-byte load; otherwise
// two loads.  Every load is issued unconditionally and masked through the
// out-of-range offset (rows at or beyond n, steps past q1).  Operands live in
// a ring of NS register sets, loads NS - 1 steps ahead of the MFMAs.  The
// complex types keep the imaginary parts in aci; for Upper their arithmetic
// runs on the stored values, conj(S) and conj(L), which gives conj(P): the
// stored form of P, as it is written back to the matrix; the block for LDS is
// conjugated.
template <typename T, bool UPPER, bool PAIRED, int GW, int MAXS_, int NCB_ = 2>
struct PanelGemm {
    using R = typename Traits<T>::R;
    static constexpr bool CPLX = Traits<T>::cplx;
    using M = Mfma<R>;
    using v4 = typename M::v4;
    static constexpr uint32_t S = sizeof(T);
    static constexpr int MAXS = MAXS_;   // superblocks per pass
    static constexpr int NCB = NCB_;     // column tiles: 2 for 32 columns, 4 for 64
    // ring depth: as deep as 256 registers allow next to the accumulators
    static constexpr int NS = NCB == 4 ? 4 : (NCB + 2 * MAXS) <= 4 ? (CPLX ? (sizeof(R) == 8 ? 4 : 5) : 8)
                                                    : (CPLX ? 4 : (sizeof(R) == 8 ? 5 : 6));
    v4 acc[MAXS][2][NCB], aci[MAXS][2][NCB];
    // column of register r of column tile cb (lane group g)
    static __device__ __forceinline__ int col_of(int r, int g, int cb) {
        return 32 * (cb >> 1) + 2 * M::row(r, g) + (cb & 1);
    }

    __amdgpu_buffer_rsrc_t rs;
    uint32_t ld;
    int n, kp, RS, sb0, l16, g;

    __device__ __forceinline__ int sb_of(int s) const { return sb0 + GW * s; }

    __device__ __forceinline__ uint32_t off(int row, int col) const {
        return UPPER ? (uint32_t(row) * ld + uint32_t(col)) * S : (uint32_t(col) * ld + uint32_t(row)) * S;
    }
    __device__ __forceinline__ void negate_all() {
        static_for<0, MAXS>([&](auto ss) {
            static_for<0, 2>([&](auto ee) {
                static_for<0, NCB>([&](auto cc) {
                    acc[ss][ee][cc] = -acc[ss][ee][cc];
                    if constexpr (CPLX) aci[ss][ee][cc] = -aci[ss][ee][cc];
                });
            });
        });
    }
    // accumulators from S(kp:n, kp:kp+w) (referenced part only): tile (s, e, cb),
    // register r holds column c = 2 row(r, g) + cb, row i = 32 sb + 2 l16 + e
    __device__ __forceinline__ void begin(int w) {
        static_for<0, MAXS>([&](auto ss) {
            constexpr int s = ss;
            const int sb = sb_of(s);
            static_for<0, 2>([&](auto ee) {
                static_for<0, NCB>([&](auto cc) {
                    static_for<0, 4>([&](auto rr) {
                        constexpr int e = ee, cb = cc, r = rr;
                        const int c = col_of(r, g, cb);
                        const int i = 32 * sb + 2 * l16 + e;
                        const bool ref = sb < RS && kp + i < n && c < w && i >= c;
                        const T x = buf_load<T>(rs, ref ? off(kp + i, kp + c) : kBufOOB);
                        acc[s][e][cb][r] = re(x);
                        if constexpr (CPLX) aci[s][e][cb][r] = x.im;
                    });
                });
            });
        });
    }
    // adds L(kp:n, q0:q1) L(kp:kp+w, q0:q1)^H (q0, q1 multiples of 4); FIRST:
    // the accumulators still hold S (begin() just issued its loads) and are
    // turned into -S once the first operand loads are in flight
    template <bool FIRST>
    __device__ __forceinline__ void accumulate(int q0, int q1) {
        if (q1 <= q0 || sb0 >= RS) {   // nothing to add, or no superblock on this wave
            if constexpr (FIRST) negate_all();
            return;
        }
        T opa[NS][NCB], opb[NS][MAXS][2];
        // A masked lane gets bit 31 set in its offset, which puts it out of the
        // buffer's range (no memory access, the load returns 0).  The mask is
        // applied arithmetically, from a value the optimiser cannot see
        // through: as a select it would be turned into a branch around the
        // load, and a branch between a load and its use drains the wait
        // counters.
        auto masked = [&](uint32_t o, bool ok) __attribute__((always_inline)) {
            uint32_t bad = ok ? 0u : 1u;
            asm volatile("" : "+v"(bad));
            return o | (bad << 31);
        };
        auto load_pair = [&](int row, int col, bool live, T& x, T& y) __attribute__((always_inline)) {
            if constexpr (PAIRED) {
                static_assert(!CPLX && sizeof(R) == 8, "paired loads are for fp64");
                const uint32_t o = masked(off(row, col), live && row < n);
                using V = uint32_t __attribute__((ext_vector_type(4)));
                using V2 = uint32_t __attribute__((ext_vector_type(2)));
                const V v = __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0);
                x = __builtin_bit_cast(T, V2{v.x, v.y});
                y = __builtin_bit_cast(T, V2{v.z, v.w});
            } else {
                x = buf_load<T>(rs, masked(off(row, col), live && row < n));
                y = buf_load<T>(rs, masked(off(row + 1, col), live && row + 1 < n));
            }
        };
        auto load_ops = [&](int q, auto setc) __attribute__((always_inline)) {
            constexpr int st = decltype(setc)::value;
            const bool live = q < q1;
            static_for<0, NCB / 2>([&](auto hh) {
                constexpr int h = hh;
                load_pair(kp + 32 * h + 2 * l16, q + g, live, opa[st][2 * h], opa[st][2 * h + 1]);
            });
            static_for<0, MAXS>([&](auto ss) {
                constexpr int s = ss;
                const int row = kp + 32 * sb_of(s) + 2 * l16;
                load_pair(row, q + g, live, opb[st][s][0], opb[st][s][1]);
            });
        };
        auto step = [&](auto setc) __attribute__((always_inline)) {
            constexpr int st = decltype(setc)::value;
            static_for<0, MAXS>([&](auto ss) {
                constexpr int s = ss;
                if (sb_of(s) < RS) {
                    static_for<0, 2>([&](auto ee) {
                        static_for<0, NCB>([&](auto cc) {
                            constexpr int e = ee, cb = cc;
                            const T& a = opa[st][cb];
                            const T& bv = opb[st][s][e];
                            if constexpr (CPLX)
                                cmac<true>(a.re, a.im, bv.re, bv.im, acc[s][e][cb], aci[s][e][cb]);
                            else
                                acc[s][e][cb] = M::mac(a, bv, acc[s][e][cb]);
                        });
                    });
                }
            });
        };
        static_for<0, NS - 1>([&](auto ss) { load_ops(q0 + 4 * ss, ss); });
        if constexpr (FIRST) negate_all();
        for (int q = q0; q < q1; q += 4 * NS) {
            static_for<0, NS>([&](auto ss) {
                constexpr int s = ss;
                load_ops(q + 4 * (s + NS - 1), ic<(s + NS - 1) % NS>{});
                step(ss);
            });
        }
    }
    // the diagonal block (superblock 0) as P into p11
    __device__ __forceinline__ void finish_lds(T* p11, int w) {
        static_assert(NCB == 2, "32 columns");
        negate_all();
        static_for<0, 2>([&](auto ee) {
            static_for<0, 2>([&](auto cc) {
                static_for<0, 4>([&](auto rr) {
                    constexpr int e = ee, cb = cc, r = rr;
                    const int c = 2 * M::row(r, g) + cb;
                    const int i = 2 * l16 + e;
                    T val;
                    if constexpr (CPLX) val = T{acc[0][e][cb][r], UPPER ? -aci[0][e][cb][r] : aci[0][e][cb][r]};
                    else val = acc[0][e][cb][r];
                    p11[i * LDD + c] = c < w ? val : zero<T>();
                });
            });
        });
    }
    // Superblocks below the diagonal block, solved from the accumulators:
    // L21 = P21 W^H, computed as L21^T = conj(W) P21^T on MFMA with the A
    // operand from wm (wm[c' LDD + c] = conj(W(c', c))) and the B operand
    // straight from the accumulators.  Register r of tile (e, cb) of lane
    // (l16, g) holds P(i, c) at c = 2 row(r, g) + cb, four distinct c over the
    // four lane groups, so step (r, cb) of the contraction runs over those c;
    // W being lower triangular, the steps with every c >= 16 are skipped for
    // c' < 16.  For complex Upper the accumulators hold conj(P) and W takes the
    // place of conj(W), which gives conj(L21), the stored form.  The result
    // tile (e, cp) holds L21(i, c') at c' = 16 cp + row(r, g), i = 32 sb + 2 l16 + e.
    __device__ __forceinline__ void solve_store(const T* wm, int w) {
        static_assert(NCB == 2, "32 columns");
        negate_all();
        static_for<0, MAXS>([&](auto ss) {
            constexpr int s = ss;
            const int sb = sb_of(s);
            if (sb < RS) {
                static_for<0, 2>([&](auto pp) {
                    constexpr int cp = pp;
                    v4 x[2], xi[2];
                    static_for<0, 2>([&](auto ee) {
                        x[ee] = v4{R(0), R(0), R(0), R(0)};
                        xi[ee] = v4{R(0), R(0), R(0), R(0)};
                    });
                    static_for<0, 4>([&](auto rr) {
                        static_for<0, 2>([&](auto cc) {
                            constexpr int r = rr, cb = cc;
                            if constexpr (!(cp == 0 && 2 * M::row(r, 0) + cb >= 16)) {
                                const int c = 2 * M::row(r, g) + cb;
                                const T a = wm[(16 * cp + l16) * LDD + c];
                                static_for<0, 2>([&](auto ee) {
                                    constexpr int e = ee;
                                    if constexpr (CPLX)
                                        cmac<UPPER>(a.re, a.im, acc[s][e][cb][r], aci[s][e][cb][r], x[e], xi[e]);
                                    else
                                        x[e] = M::mac(a, acc[s][e][cb][r], x[e]);
                                });
                            }
                        });
                    });
                    static_for<0, 4>([&](auto rr) {
                        constexpr int r = rr;
                        const int col = 16 * cp + M::row(r, g);
                        const int row = kp + 32 * sb + 2 * l16;
                        if constexpr (PAIRED) {
                            // rows row, row + 1 of one column with one 16-byte store (n even);
                            // the elements are copied out before the bit cast (a bit cast
                            // taken of the vector element itself was compiled into a
                            // store of element 0 for every r)
                            using V = uint32_t __attribute__((ext_vector_type(4)));
                            using V2 = uint32_t __attribute__((ext_vector_type(2)));
                            const R d0 = x[0][r], d1 = x[1][r];
                            const V2 lo = __builtin_bit_cast(V2, d0), hi = __builtin_bit_cast(V2, d1);
                            const bool st = row < n && col < w;
                            __builtin_amdgcn_raw_buffer_store_b128(V{lo.x, lo.y, hi.x, hi.y}, rs,
                                                                   st ? off(row, kp + col) : kBufOOB, 0, 0);
                        } else {
                            static_for<0, 2>([&](auto ee) {
                                constexpr int e = ee;
                                T val;
                                if constexpr (CPLX) val = T{x[e][r], xi[e][r]};
                                else val = x[e][r];
                                const bool st = row + e < n && col < w;
                                buf_store<T>(rs, st ? off(row + e, kp + col) : kBufOOB, val);
                            });
                        }
                    });
                });
            }
        });
    }

    // ---- 64-column passes (real types): NCB = 4, one superblock
    // A superblock below the 64 x 64 diagonal block, solved from the
    // accumulators in two stages: L_a = P_a W1^T for the first 32 columns (as
    // solve_store), then P_b -= L_a L21'^T on MFMA with L21' (rows 32..63,
    // columns 0..31 of the diagonal block's factor) from LDS as the A operand
    // and L_a straight from the first stage's result registers as the B
    // operand: register r' of result tile (e, cp) holds L_a(i, c') at
    // c' = 16 cp + row(r', g), four distinct c' over the lane groups, so step
    // (cp, r') of that contraction runs over them.  Then L_b = P_b W2^T.
    __device__ __forceinline__ void solve_store2(const T* wm1, const T* wm2, const T* pl, int w) {
        static_assert(NCB == 4 && MAXS == 1 && !CPLX, "64 columns, real");
        negate_all();
        const int sb = sb0;
        if (sb >= RS) return;
        const int row = kp + 32 * sb + 2 * l16;
        auto store_pair = [&](int col, bool colok, R v0, R v1) __attribute__((always_inline)) {
            if constexpr (PAIRED) {
                using V = uint32_t __attribute__((ext_vector_type(4)));
                using V2 = uint32_t __attribute__((ext_vector_type(2)));
                const V2 lo = __builtin_bit_cast(V2, v0), hi = __builtin_bit_cast(V2, v1);
                const bool st = row < n && colok;
                __builtin_amdgcn_raw_buffer_store_b128(V{lo.x, lo.y, hi.x, hi.y}, rs,
                                                       st ? off(row, kp + col) : kBufOOB, 0, 0);
            } else {
                buf_store<T>(rs, row < n && colok ? off(row, kp + col) : kBufOOB, T(v0));
                buf_store<T>(rs, row + 1 < n && colok ? off(row + 1, kp + col) : kBufOOB, T(v1));
            }
        };
        // 16 columns 16 cp.. of half h: x[e] = P(half) W^T from the
        // accumulator tiles 2 h, 2 h + 1, stored
        auto part = [&](auto hh, auto pp, const T* wmh, v4 (&x)[2]) __attribute__((always_inline)) {
            constexpr int h = hh, cp = pp;
            static_for<0, 2>([&](auto ee) { x[ee] = v4{R(0), R(0), R(0), R(0)}; });
            static_for<0, 4>([&](auto rr) {
                static_for<0, 2>([&](auto cc) {
                    constexpr int r = rr, cb = cc;
                    if constexpr (!(cp == 0 && 2 * M::row(r, 0) + cb >= 16)) {
                        const int c = 2 * M::row(r, g) + cb;
                        const T a = wmh[(16 * cp + l16) * LDD + c];
                        static_for<0, 2>([&](auto ee) {
                            constexpr int e = ee;
                            x[e] = M::mac(a, acc[0][e][2 * h + cb][r], x[e]);
                        });
                    }
                });
            });
            static_for<0, 4>([&](auto rr) {
                constexpr int r = rr;
                const int col = 16 * cp + M::row(r, g);
                const R d0 = x[0][r], d1 = x[1][r];
                store_pair(32 * h + col, 32 * h + col < w, d0, d1);
            });
        };
        // the first half, each 16-column group applied to P_b as soon as it
        // is solved: P_b -= L_a(:, group) L21'(:, group)^T
        static_for<0, 2>([&](auto pp) {
            constexpr int cp = pp;
            v4 x[2];
            part(ic<0>{}, ic<cp>{}, wm1, x);
            static_for<0, 4>([&](auto rr) {
                constexpr int r = rr;
                const int cpr = 16 * cp + M::row(r, g);
                static_for<0, 2>([&](auto cc) {
                    constexpr int cb = cc;
                    const T a = -pl[(2 * l16 + cb) * LDD + cpr];
                    static_for<0, 2>([&](auto ee) {
                        constexpr int e = ee;
                        acc[0][e][2 + cb] = M::mac(a, x[e][r], acc[0][e][2 + cb]);
                    });
                });
            });
        });
        static_for<0, 2>([&](auto pp) {
            v4 x[2];
            part(ic<1>{}, pp, wm2, x);
        });
    }
};

// One matrix, panel by panel.  Per panel k:
//
//   wave 0:     GEMM of the diagonal block -> p11 (LDS); factor it, L11 to
//               the matrix, the inverse W of L11 to LDS
//   waves 1..3: GEMM of the first superblocks below (sb = w + 3 s, s < CH),
//               kept in the accumulators
//   sync
//   waves 1..3: solve those from the accumulators, L21 to the matrix
//   all waves:  the remaining superblocks, round-robin, CH at a time: GEMM,
//               solve from the accumulators, L21 to the matrix
//   sync
//
// P never leaves the registers, so the traffic per panel is S and the
// columns of L left of k read, and L21 written.  The one-wave factorisation
// overlaps the first GEMMs of the other three waves, and the workgroup is
// small (four waves, under 40 KB of LDS), so that two matrices share a
// compute unit and fill each other's gaps.
template <typename T, bool UPPER, bool PAIRED>
__device__ __forceinline__ void factor_matrix(__amdgpu_buffer_rsrc_t rs, uint32_t ld, int n,
                                              int wave, T* p11, T* wm,
                                              typename FactorType<T>::type* colx,
                                              typename Traits<typename FactorType<T>::type>::R* rdiag,
                                              int32_t* s_inf)
{
    using R = typename Traits<T>::R;
    constexpr bool CPLX = Traits<T>::cplx;
    constexpr int GW = WAVES - 1;                          // waves beside the factoring one
    constexpr int CH = (CPLX && sizeof(R) == 8) ? 1 : 2;   // superblocks per pass
    // The lane index is re-read at every phase and hidden from the optimiser,
    // so that addresses derived from it are recomputed where they are used
    // instead of being hoisted and kept live (in registers) across phases.
    auto lane_now = [&]() __attribute__((always_inline)) {
        int lane = threadIdx.x & 63;
        asm volatile("" : "+v"(lane));
        return lane;
    };
    auto setup = [&](auto& gm, int k, int RS, int sb0) __attribute__((always_inline)) {
        const int lane = lane_now();
        gm.rs = rs;
        gm.ld = ld;
        gm.n = n;
        gm.kp = k;
        gm.RS = RS;
        gm.sb0 = sb0;
        gm.l16 = lane & 15;
        gm.g = lane >> 4;
    };
    // the superblocks from 3 CH + 1 on, after the sync
    auto rest = [&](int k, int w, int RS) __attribute__((always_inline)) {
        using G4 = PanelGemm<T, UPPER, PAIRED, WAVES, CH>;
        for (int sb = GW * CH + 1 + wave; sb < RS; sb += WAVES * CH) {
            G4 gm;
            setup(gm, k, RS, sb);
            gm.begin(w);
            gm.template accumulate<true>(0, k);
            gm.solve_store(wm, w);
        }
    };
    if (wave == 0) {
        using G1 = PanelGemm<T, UPPER, PAIRED, 1, 1>;
        for (int k = 0; k < n; k += NBP) {
            const int w = min(NBP, n - k);
            const int RS = (n - k + 31) >> 5;
            {
                G1 gd;
                setup(gd, k, 1, 0);
                gd.begin(w);
                gd.template accumulate<true>(0, k);
                gd.finish_lds(p11, w);
            }
            wave_lds_sync();
            {
                const int lane = lane_now();
                if constexpr (CPLX) factor_invert_inplace<T, UPPER>(p11, wm, rdiag, lane, k, n, w, rs, ld, *s_inf);
                else factor_diag<T, UPPER>(p11, wm, colx, rdiag, lane, k, n, w, rs, ld, *s_inf);
            }
            __syncthreads();
            rest(k, w, RS);
            __syncthreads();
        }
    } else {
        using G3 = PanelGemm<T, UPPER, PAIRED, GW, CH>;
        for (int k = 0; k < n; k += NBP) {
            const int w = min(NBP, n - k);
            const int RS = (n - k + 31) >> 5;
            G3 gm;
            setup(gm, k, RS, wave);
            const bool mine = wave < RS;
            if (mine) {
                gm.begin(w);
                gm.template accumulate<true>(0, k);
            }
            __syncthreads();
            if (mine) gm.solve_store(wm, w);
            rest(k, w, RS);
            __syncthreads();
        }
    }
}

// Real types: 64-column panels.  The left-looking GEMM streams the columns
// of L left of k once per panel, so twice the panel width halves that
// traffic.  The 64 x 64 diagonal block is three 32 x 32 GEMM units (D11 =
// rows 0..31 x columns 0..31, D21 = rows 32..63 x columns 0..31, D22 = rows
// 32..63 x columns 32..63, all over the columns of L left of k) and two
// 32 x 32 factorisations.  Per panel k (64 columns):
//
//   waves 1..3: D11 -> p11, D21 -> pa, D22 -> p22
//   sync
//   wave 0:     factor P11 (L11, W1); L21' = P21' W1^T on MFMA (to the
//               matrix and to pl); P22 -= L21' L21'^T on MFMA; factor P22
//               (L22, W2)
//   waves 1..3: GEMM of superblocks w + 1 and w + 4, kept in the
//               accumulators
//   sync
//   waves 1..3: solve the kept superblocks from the accumulators in two
//               stages (solve_store2)
//   all waves:  the remaining superblocks, each taken by the next wave free:
//               GEMM, two-stage solve
//   sync
template <typename T, bool UPPER, bool PAIRED>
__device__ __forceinline__ void factor_matrix_wide(__amdgpu_buffer_rsrc_t rs, uint32_t ld, int n,
                                                   int wave, T* p11, T* wm1, T* pa, T* p22, T* pl,
                                                   T* wm2, double* colx, double* rdiag,
                                                   int32_t* s_inf, int32_t* ctr)
{
    using R = typename Traits<T>::R;
    using M = Mfma<R>;
    using v4 = typename M::v4;
    static_assert(!Traits<T>::cplx, "real types");
    constexpr uint32_t S = sizeof(T);
    auto off = [&](int row, int col) -> uint32_t {
        return UPPER ? (uint32_t(row) * ld + uint32_t(col)) * S : (uint32_t(col) * ld + uint32_t(row)) * S;
    };
    auto lane_now = [&]() __attribute__((always_inline)) {
        int lane = threadIdx.x & 63;
        asm volatile("" : "+v"(lane));
        return lane;
    };
    auto setup = [&](auto& gm, int k, int RS, int sb0) __attribute__((always_inline)) {
        const int lane = lane_now();
        gm.rs = rs;
        gm.ld = ld;
        gm.n = n;
        gm.kp = k;
        gm.RS = RS;
        gm.sb0 = sb0;
        gm.l16 = lane & 15;
        gm.g = lane >> 4;
    };
    using G1 = PanelGemm<T, UPPER, PAIRED, 1, 1>;
    using G64 = PanelGemm<T, UPPER, PAIRED, 1, 1, 4>;
    // a 32 x 32 unit of the diagonal block: rows 32 sb.. of the panel at kp,
    // its columns 0..31, over the columns of L left of q1, into dst
    auto unit = [&](int kp, int RS, int sb, int w, int q1, T* dst) __attribute__((always_inline)) {
        G1 gd;
        setup(gd, kp, RS, sb);
        gd.begin(w);
        gd.template accumulate<true>(0, q1);
        gd.finish_lds(dst, w);
    };
    // the superblocks from 8 on, each taken by the next wave free (the waves
    // that solve kept superblocks first come later): an LDS counter, reset by
    // wave 0 between the syncs before this phase
    auto rest = [&](int k, int w, int RS) __attribute__((always_inline)) {
        for (;;) {
            int j = 0;
            if (lane_now() == 0) j = atomicAdd(ctr, 1);
            const int sb = 8 + __builtin_amdgcn_readlane(j, 0);
            if (sb >= RS) break;
            G64 gm;
            setup(gm, k, RS, sb);
            gm.begin(w);
            gm.template accumulate<true>(0, k);
            gm.solve_store2(wm1, wm2, pl, w);
        }
    };
    // (each role runs its own copy of the panel loop with the same syncs: in
    // one loop the compiler keeps the roles' values live together)
    if (wave == 0) {
        for (int k = 0; k < n; k += 2 * NBP) {
            const int w = min(2 * NBP, n - k);
            const int wa = min(NBP, w), wb = w - NBP;    // wb <= 0: no second half
            const int RS = (n - k + 31) >> 5;
            __syncthreads();
            if (lane_now() == 0) *ctr = 0;
            factor_diag<T, UPPER>(p11, wm1, colx, rdiag, lane_now(), k, n, wa, rs, ld, *s_inf);
            if (wb > 0) {
                wave_lds_sync();
                const int lane = lane_now();
                const int l16 = lane & 15, g = lane >> 4;
                // L21' = P21' W1^T (both operands from LDS), to the matrix and to pl
                static_for<0, 2>([&](auto bb) {
                    constexpr int ib = bb;
                    static_for<0, 2>([&](auto pp) {
                        constexpr int cbp = pp;
                        v4 x = {R(0), R(0), R(0), R(0)};
                        static_for<0, 4 * (cbp + 1)>([&](auto uu) {   // W1 is lower triangular
                            constexpr int u = uu;
                            const int c = 4 * u + g;
                            x = M::mac(pa[(ib * 16 + l16) * LDD + c], wm1[(cbp * 16 + l16) * LDD + c], x);
                        });
                        static_for<0, 4>([&](auto rr) {
                            constexpr int r = rr;
                            const int i = ib * 16 + M::row(r, g);
                            const int c = cbp * 16 + l16;
                            const T v = x[r];
                            pl[i * LDD + c] = v;
                            const bool st = k + NBP + i < n && c < wa;
                            buf_store<T>(rs, st ? off(k + NBP + i, k + c) : kBufOOB, v);
                        });
                    });
                });
                wave_lds_sync();
                // P22 -= L21' L21'^T (lower tiles)
                static_for<0, 3>([&](auto tt) {
                    constexpr int mt = tt == 0 ? 0 : 1, nt = tt == 2 ? 1 : 0;
                    v4 x = {R(0), R(0), R(0), R(0)};
                    static_for<0, NBP / 4>([&](auto uu) {
                        constexpr int u = uu;
                        const int c = 4 * u + g;
                        x = M::mac(pl[(16 * mt + l16) * LDD + c], pl[(16 * nt + l16) * LDD + c], x);
                    });
                    static_for<0, 4>([&](auto rr) {
                        constexpr int r = rr;
                        T& d = p22[(16 * mt + M::row(r, g)) * LDD + 16 * nt + l16];
                        d = d - T(x[r]);
                    });
                });
                wave_lds_sync();
                factor_diag<T, UPPER>(p22, wm2, colx, rdiag, lane_now(), k + NBP, n, wb, rs, ld, *s_inf);
            }
            __syncthreads();
            rest(k, w, RS);
            __syncthreads();
        }
    } else {
        for (int k = 0; k < n; k += 2 * NBP) {
            const int w = min(2 * NBP, n - k);
            const int wa = min(NBP, w), wb = w - NBP;
            const int RS = (n - k + 31) >> 5;
            if (wave == 1) unit(k, 1, 0, wa, k, p11);                       // D11
            else if (wb > 0) {
                if (wave == 2) unit(k, 2, 1, wa, k, pa);                    // D21
                else unit(k + NBP, 1, 0, wb, k, p22);                       // D22
            }
            __syncthreads();
            {
                G64 gm, gn;
                setup(gm, k, RS, wave + 1);
                setup(gn, k, RS, wave + 4);
                const bool mine = wave + 1 < RS, next = wave + 4 < RS;
                if (mine) {
                    gm.begin(w);
                    gm.template accumulate<true>(0, k);
                }
                if (next) {
                    gn.begin(w);
                    gn.template accumulate<true>(0, k);
                }
                __syncthreads();
                if (mine) gm.solve_store2(wm1, wm2, pl, w);
                if (next) gn.solve_store2(wm1, wm2, pl, w);
            }
            rest(k, w, RS);
            __syncthreads();
        }
    }
}

// LDS: the diagonal block P11 (then L11), conj of the inverse of L11, the
// pivot exchange, 1 / L(j, j) and the info word
template <typename T>
struct Smem {
    using C = typename FactorType<T>::type;
    using Rc = typename Traits<C>::R;
    static constexpr int WIDE = Traits<T>::cplx ? 1 : NBP * LDD;   // 64-column panels (real types)
    T p11[NBP * LDD];
    T wm[NBP * LDD];
    T pa[WIDE], p22[WIDE], pl[WIDE], wm2[WIDE];
    C colx[2 * NBP];
    Rc rdiag[NBP];
    int32_t inf;
    int32_t ctr;   // superblocks taken (64-column panels)
};

template <typename T, bool UPPER>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2)))
void potrf_blocked_kernel(T* __restrict__ A, int n, int64_t lda, int64_t stride, int64_t batch,
                          int32_t* __restrict__ info)
{
    using R = typename Traits<T>::R;
    constexpr bool CPLX = Traits<T>::cplx;
    __shared__ __attribute__((aligned(16))) Smem<T> sm;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t ld = uint32_t(lda);
    for (int64_t b = blockIdx.x; b < batch; b += gridDim.x) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(A + b * stride);
        if (threadIdx.x == 0) sm.inf = 0;
        // (the paired 16-byte loads are used for fp64 Lower with n even; the
        // fp32 pairs gave wrong results on the GPU and are not used)
        if constexpr (CPLX) {
            factor_matrix<T, UPPER, false>(rs, ld, n, wave, sm.p11, sm.wm, sm.colx, sm.rdiag, &sm.inf);
        } else if constexpr (!UPPER && sizeof(R) == 8) {
            if ((n & 1) == 0)
                factor_matrix_wide<T, UPPER, true>(rs, ld, n, wave, sm.p11, sm.wm, sm.pa, sm.p22, sm.pl, sm.wm2,
                                                   sm.colx, sm.rdiag, &sm.inf, &sm.ctr);
            else
                factor_matrix_wide<T, UPPER, false>(rs, ld, n, wave, sm.p11, sm.wm, sm.pa, sm.p22, sm.pl, sm.wm2,
                                                    sm.colx, sm.rdiag, &sm.inf, &sm.ctr);
        } else {
            factor_matrix_wide<T, UPPER, false>(rs, ld, n, wave, sm.p11, sm.wm, sm.pa, sm.p22, sm.pl, sm.wm2,
                                                sm.colx, sm.rdiag, &sm.inf, &sm.ctr);
        }
        if (threadIdx.x == 0 && info != nullptr) info[b] = sm.inf;
        __syncthreads();
    }
}

// ---------------------------------------------------------------- host side
constexpr int64_t kMaxGrid = int64_t(1) << 20;

template <typename T>
bool supported_t(int n, int64_t lda) {
    return n >= 1 && n <= Shape<T>::MAXN && lda * int64_t(n) * int64_t(sizeof(T)) < (int64_t(1) << 31);
}

template <typename T>
bool geometry_t(int n, int64_t batch, Geometry& g) {
    if (n < 1 || n > Shape<T>::MAXN) return false;
    g.family = FAM_BLOCKED;
    g.P = g.R = g.G = 0;
    g.threads = 64 * WAVES;
    g.panel = Traits<T>::cplx ? NBP : 2 * NBP;   // real types: 64-column panels
    g.grid = batch < kMaxGrid ? batch : kMaxGrid;
    g.lds = int64_t(sizeof(Smem<T>));
    return true;
}

template <typename T>
hipError_t potrf_t(bool upper, int n, void* A, int64_t lda, int64_t stride, int64_t batch,
                   int32_t* info, hipStream_t s) {
    const dim3 gd((unsigned)(batch < kMaxGrid ? batch : kMaxGrid)), bd(64 * WAVES);
    T* a = static_cast<T*>(A);
    if (upper) return launch(potrf_blocked_kernel<T, true>, gd, bd, 0, s, a, n, lda, stride, batch, info);
    return launch(potrf_blocked_kernel<T, false>, gd, bd, 0, s, a, n, lda, stride, batch, info);
}

}  // namespace blocked_detail
}  // namespace bl
