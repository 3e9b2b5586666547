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

// Wavefronts per workgroup (each independent).  One: a finished wavefront's
// slot takes the next workgroup at once, where a wider workgroup would hold its
// slots until its slowest wavefront ends (at one wavefront per SIMD, the 64 x 1
// window ran 15% slower with four per workgroup).
constexpr int kTinyWaves = 1;

// At most this many workgroups per launch: a dispatch counts its work-items in
// 32 bits, and a batch of 2^30 matrices of order <= 4 would need 2^26 one-wave
// workgroups.  Larger batches run as several launches over consecutive slices.
constexpr int64_t kTinyMaxGrid = int64_t(1) << 24;

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
            const uint32_t off = (k < nrhs) ? boff[r] : kBufOOB;
            y[r][k] = buf_load<T>(rb, off, uint32_t(k) * ldb_b);
            yf[r][k] = zero<T>();
        });
    });
    // forward: L y = b, p ascending
    static_for<0, NB>([&](auto pp) {
        constexpr int pv = pp;
        constexpr int rp = pv / P;
        uint32_t* row = ldsw + (pv & 1) * parity_words + p * roww;
        const bool owner = q == pv % P;
        T yp[NRHS];
        if constexpr (P == 16 && std::is_same<T, float>::value) {
            // a partition is one DPP row: the owner's value by a row broadcast
            static_for<0, NRHS>([&](auto kk) {
                constexpr int k = kk;
                const T v = scale(y[rp][k], invd[rp]);
                yf[rp][k] = select(owner, v, yf[rp][k]);
                yp[k] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                    0, __builtin_bit_cast(int, v), 0x150 + (pv % 16), 0xf, 0xf, false));
            });
        } else {
            static_for<0, NRHS>([&](auto kk) {
                constexpr int k = kk;
                const T v = scale(y[rp][k], invd[rp]);
                yf[rp][k] = select(owner, v, yf[rp][k]);
                if (owner) lds_put<T>(row, NB + 1 + k, v);
            });
            wave_lds_sync();
            static_for<0, NRHS>([&](auto kk) { yp[kk] = lds_get<T>(row, NB + 1 + kk); });
        }
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
            const uint32_t off = (inf == 0 && k < nrhs) ? boff[r] : kBufOOB;
            buf_store<T>(rb, off, xf[r][k], uint32_t(k) * ldb_b);
        });
    });
}

// x as held by lane src (src wave-uniform)
template <typename T>
__device__ __forceinline__ T lane_read(const T& x, int src) {
    uint32_t w[words<T>()];
    __builtin_memcpy(w, &x, sizeof(T));
    static_for<0, words<T>()>([&](auto ii) { w[ii] = __builtin_amdgcn_readlane(w[ii], src); });
    T y;
    __builtin_memcpy(&y, w, sizeof(T));
    return y;
}

// The column recurrence on the rows a lane holds (rows i = q + r P of the
// matrix of partition p), with the pivot columns exchanged through xbuf
// (two parity buffers of PARTS rows of ROWW words).  On return a holds the
// factor's rows, invd 1 / L(i, i) (posv only) and inf the first failing column.
//
// Register slots a[r][k] with k > i (the row's upper part) are scratch: they
// absorb updates but never feed a referenced slot, so a step needs no
// per-row guards.  Rows at or beyond n hold the identity, so every one of
// the NB steps can run unconditionally: a padding step sees d = 1 and
// leaves the referenced part alone.  After a failed pivot the recurrence
// continues (NaN from the failing column on); the leading columns are final
// by then and info keeps the first failing column.
    //
// Look-ahead: within step j, column j+1 is updated first and published to
// LDS before the rest of step j's updates, so the exchange latency hides
// behind that arithmetic.  Column j is published at slots relative to j
// (row i -> slot i - j), so the entries a step needs always start at slot
// 0; a step reads them from LDS where it uses them (broadcast reads), so no
// copy of the column is held in registers.  Rows above j write to a spare
// slot at NB.
// The pivot terms of a step: from one reciprocal square root (pivot_terms)
// where ONE_RSQ, else from three separate quarter-rate instructions.  Which is
// faster depends on the window: the single one shortens the step, but the
// compiler then schedules the window with more registers, and for the n = 33
// window (11 x 3) that costs a wavefront per SIMD (measured 43.4 against 42.6
// us at b16384), while the n = 17 window gains (24.4 against 25.8 us).
template <bool ONE_RSQ, typename Rt>
__device__ __forceinline__ void step_pivot(Rt d, Rt& inv, Rt& rs, Rt& sq) {
    if constexpr (ONE_RSQ) {
        pivot_terms(d, inv, rs, sq);
    } else {
        inv = pivot_rcp(d);
        rs = pivot_rsq(d);
        sq = pivot_sqrt(d);
    }
}

template <typename T, int P, int R, bool UPPER, int NRHS, int ROWW, bool ONE_RSQ>
__device__ __forceinline__ void factor_rows(T (&a)[R][P * R], typename Traits<T>::R (&invd)[R],
                                            uint32_t* xbuf, int p, int q, int32_t& inf)
{
    using Rt = typename Traits<T>::R;
    constexpr int NB = P * R;
    constexpr int PARTS = 63 / P + 1;
    auto xrow = [&](int par, int part) -> uint32_t* { return xbuf + (par * PARTS + part) * ROWW; };
    auto publish = [&](auto jc) {
        constexpr int j = decltype(jc)::value;
        constexpr int rj = j / P;
        uint32_t* row = xrow(j & 1, p);
        static_for<rj, R>([&](auto rr) {
            constexpr int r = rr;
            const int i = q + r * P;
            const int slot = (r == rj) ? ((i >= j) ? i - j : NB) : i - j;
            lds_put<T>(row, slot, a[r][j]);
        });
    };
    // entry for row k of column j (k >= j), read from the published column
    // (the buffer of column j is not overwritten before step j + 2)
    auto colv = [&](int j, int k) -> T { return lds_get<T>(xrow(j & 1, p), k - j); };

    inf = 0;
    static_for<0, R>([&](auto rr) { invd[rr] = Rt(1); });
    publish(ic<0>{});
    wave_lds_sync();
    static_for<0, NB>([&](auto jj) {
        constexpr int j = jj;
        constexpr int rj = j / P;
        const Rt d = re(colv(j, j));
        inf = (inf == 0 && !(d > Rt(0))) ? (j + 1) : inf;
        Rt inv, rs, sq;
        step_pivot<ONE_RSQ>(d, inv, rs, sq);
        T t[R];
        static_for<rj, R>([&](auto rr) {
            constexpr int r = rr;
            t[r] = scale(a[r][j], inv);
        });
        if constexpr (j + 1 < NB) {
            constexpr int rn = (j + 1) / P;
            const T cj1 = colv(j, j + 1);
            static_for<rn, R>([&](auto rr) {
                constexpr int r = rr;
                sub_mul_conj(a[r][j + 1], t[r], cj1);
            });
            publish(ic<j + 1>{});
            wave_lds_sync();
        }
        static_for<rj, R>([&](auto rr) {
            constexpr int r = rr;
            constexpr int kend = cmin(NB, (r + 1) * P);
            static_for<j + 2, kend>([&](auto kk) {
                constexpr int k = kk;
                sub_mul_conj(a[r][k], t[r], colv(j, k));
            });
            if constexpr (r == rj) {
                // the one row block that holds row j itself
                const bool diag = (q + r * P) == j;
                a[r][j] = select(diag, diag_value<T>(sq, UPPER), scale(a[r][j], rs));
                if constexpr (NRHS > 0) invd[r] = diag ? rs : invd[r];
            } else {
                a[r][j] = scale(a[r][j], rs);
            }
        });
    });

}

// The same recurrence for fp32 partitions of exactly 16 lanes (P = 16): a
// partition is one DPP row, so the entry of row k = k' + 16 r of column j sits
// in register a[r][j] of lane k' of the same row and reaches every lane of the
// matrix by a DPP row broadcast: the pivot by a broadcast move, every update
// by a broadcast inside its multiply-add.  No LDS exchange, so no round trip
// per step.  Register slots right of a row's diagonal are scratch, as in
// factor_rows.
template <typename T, int R, bool UPPER, int NRHS, bool ONE_RSQ>
__device__ __forceinline__ void factor_rows_dpp(T (&a)[R][16 * R], float (&invd)[R], int q, int32_t& inf)
{
    static_assert(std::is_same<T, float>::value, "fp32 partitions of 16 lanes");
    constexpr int NB = 16 * R;
    inf = 0;
    static_for<0, R>([&](auto rr) { invd[rr] = 1.0f; });
    static_for<0, NB>([&](auto jj) {
        constexpr int j = jj;
        constexpr int rj = j / 16;
        const float d = __builtin_bit_cast(
            float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a[rj][j]), 0x150 + (j % 16), 0xf,
                                               0xf, false));
        inf = (inf == 0 && !(d > 0.0f)) ? (j + 1) : inf;
        float inv, rs, sq;
        step_pivot<ONE_RSQ>(d, inv, rs, sq);
        float nt[R];
        static_for<rj, R>([&](auto rr) {
            constexpr int r = rr;
            nt[r] = -(a[r][j] * inv);
        });
        // column j + 1 first (the next pivot's entry), then the rest
        if constexpr (j + 1 < NB) {
            constexpr int k = j + 1;
            static_for<k / 16, R>([&](auto rr) {
                constexpr int r = rr;
                fma_bcast16<k % 16, r == k / 16>(a[r][k], nt[r], a[k / 16][j]);
            });
        }
        static_for<rj, R>([&](auto rr) {
            constexpr int r = rr;
            constexpr int kend = cmin(NB, (r + 1) * 16);
            static_for<j + 2, kend>([&](auto kk) {
                constexpr int k = kk;
                // (wait states before the first read of each source register)
                fma_bcast16<k % 16, k == j + 2 || k % 16 == 0>(a[r][k], nt[r], a[k / 16][j]);
            });
        });
        // column j is the broadcast source of every row block's updates, so it
        // is scaled only once they are all issued
        static_for<rj, R>([&](auto rr) {
            constexpr int r = rr;
            if constexpr (r == rj) {
                const bool diag = (q + r * 16) == j;
                a[r][j] = diag ? diag_value<T>(sq, UPPER) : a[r][j] * rs;
                if constexpr (NRHS > 0) invd[r] = diag ? rs : invd[r];
            } else {
                a[r][j] = a[r][j] * rs;
            }
        });
    });
}

// The same recurrence with one matrix per wavefront (P = 64, R = 1: lane i
// holds row i), arranged so that its latencies overlap.  The pivot and the
// entry S(j + 1, j) are read from lanes j and j + 1 directly, without the LDS
// round trip.  Step j + 1's pivot,
// reciprocals and scaled entries are computed in step j, as soon as column
// j + 1 is final.  The broadcast reads of the published column go in chunks of
// 64 bytes, each issued one chunk ahead of the updates that use it, with
// scheduling fences between chunks: left to itself the scheduler issues each
// read just before its use and then waits for it, one LDS round trip per
// read.  The exchange buffer layout and the scratch slots are those of
// factor_rows.
template <typename T, bool UPPER, int NRHS, int ROWW, bool ONE_RSQ>
__device__ __forceinline__ void factor_rows_lane(T (&a)[1][64], typename Traits<T>::R (&invd)[1],
                                                 uint32_t* xbuf, int q, int32_t& inf)
{
    using Rt = typename Traits<T>::R;
    constexpr int NB = 64;
    constexpr int CH = 64 / int(sizeof(T));     // column entries per chunk
    auto xrow = [&](int par) -> uint32_t* { return xbuf + par * ROWW; };
    auto publish = [&](auto jc) {
        constexpr int j = decltype(jc)::value;
        lds_put<T>(xrow(j & 1), q >= j ? q - j : NB, a[0][j]);
    };

    inf = 0;
    invd[0] = Rt(1);
    publish(ic<0>{});
    wave_lds_sync();
    Rt d = re(lane_read(a[0][0], 0));
    Rt inv, rs, sq;
    step_pivot<ONE_RSQ>(d, inv, rs, sq);
    T t = scale(a[0][0], inv);
    static_for<0, NB>([&](auto jj) {
        constexpr int j = jj;
        // entries k = j + 2 .. NB - 1 of column j sit at slots s = k - j;
        // chunk c holds slots [c CH, (c + 1) CH)
        constexpr int NC = (NB - j + CH - 1) / CH;
        constexpr bool BULK = j + 2 < NB;
        const uint32_t* col = xrow(j & 1);
        T cv[2][CH];
        auto fetch = [&](auto cc) {
            constexpr int c = cc;
            static_for<cmax(2, c * CH), cmin((c + 1) * CH, NB - j)>([&](auto ss) {
                constexpr int sl = ss;
                cv[c & 1][sl - c * CH] = lds_get<T>(col, sl);
            });
        };
        auto apply = [&](auto cc) {
            constexpr int c = cc;
            static_for<cmax(2, c * CH), cmin((c + 1) * CH, NB - j)>([&](auto ss) {
                constexpr int sl = ss;
                sub_mul_conj(a[0][j + sl], t, cv[c & 1][sl - c * CH]);
            });
        };
        if constexpr (BULK) fetch(ic<0>{});
        inf = (inf == 0 && !(d > Rt(0))) ? (j + 1) : inf;
        Rt d_n = d, inv_n = inv, rs_n = rs, sq_n = sq;
        T t_n = t;
        if constexpr (j + 1 < NB) {
            // column j + 1 first: it feeds the next pivot and the next exchange
            sub_mul_conj(a[0][j + 1], t, lane_read(a[0][j], j + 1));
            publish(ic<j + 1>{});
            wave_lds_sync();
            d_n = re(lane_read(a[0][j + 1], j + 1));
            step_pivot<ONE_RSQ>(d_n, inv_n, rs_n, sq_n);
            t_n = scale(a[0][j + 1], inv_n);
        }
        const bool diag = q == j;
        a[0][j] = select(diag, diag_value<T>(sq, UPPER), scale(a[0][j], rs));
        if constexpr (NRHS > 0) invd[0] = diag ? rs : invd[0];
        if constexpr (BULK) {
            static_for<0, NC>([&](auto cc) {
                constexpr int c = cc;
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (c + 1 < NC) fetch(ic<c + 1>{});
                apply(cc);
            });
            __builtin_amdgcn_sched_barrier(0);
        }
        d = d_n;
        inv = inv_n;
        rs = rs_n;
        sq = sq_n;
        t = t_n;
    });
}

// Packed path: each matrix's image in LDS starts at a multiple of IMGP
// elements, IMGP >= n*n with IMGP = P (mod 32), so that the partitions of a
// wave read from different LDS banks.
template <int P, int R>
constexpr int packed_pitch() {
    return (P * R) * (P * R) + (((P - (P * R) * (P * R)) % 32) + 32) % 32;
}
// Words of LDS for the image: every partition (the dead tail one included)
// plus one more matrix, where steps past the run land.
template <typename T, int P, int R>
constexpr int packed_image_words() {
    return (63 / P + 2) * packed_pitch<P, R>() * words<T>();
}
// Upper with one matrix per wavefront (P = 64, R = 1, potrf): lane i's row is
// column i of A, so per-row loads would have every instruction touch 64
// cache lines, one element each, and with several wavefronts per CU the lines
// leave the L1 cache before their other elements are read.  Instead the
// matrix moves through LDS in slabs of SR rows of A, SR elements being one
// 128-byte line of a column: lane l carries element (c0 + l mod SR,
// u (64 / SR) + l / SR) of instruction u, so each instruction covers whole
// lines, and the slab is transposed through a tile of 64 columns with a pitch
// of one line plus 16 bytes.
template <typename T, int P, int R, bool UPPER, int NRHS, bool PACKED>
constexpr bool use_slabs() { return UPPER && P == 64 && R == 1 && NRHS == 0 && !PACKED; }
template <typename T> constexpr int slab_rows() { return 128 / int(sizeof(T)); }
template <typename T> constexpr int slab_pitch_words() { return slab_rows<T>() * words<T>() + 4; }
template <typename T> constexpr int slab_tile_words() { return 64 * slab_pitch_words<T>(); }

// Where the packed path is used (fp32 only), from timings of both variants on
// MI355X over orders 8..33.  Lower: the rows of one column are contiguous,
// so the per-row loads are already coalesced over a lane group, and the
// packed path only wins for the smallest windows (order <= 12).  Upper: a
// lane's row is a column of A, the per-row loads are strided across lanes,
// and the packed path wins while its image stays small (<= 12 KiB per wave,
// orders up to 18); beyond that the image limits the wavefronts per CU.
constexpr int kPackedLowerMaxOrder = 12;
constexpr int kPackedUpperMaxBytes = 12 * 1024;

// Windows whose steps take their pivot terms from one reciprocal square root
// (measured on MI355X; the others keep three separate instructions): the
// n = 17 window (17 x 1), the one-matrix-per-wavefront windows (64 x 1) and
// the fused posv window of orders 25..32 (16 x 2).
template <typename T, int P, int R, int NRHS>
constexpr bool one_rsq_window() {
    constexpr bool f32 = std::is_same<T, float>::value;
    return (f32 && P == 17 && R == 1) || (P == 64 && R == 1) ||
           (f32 && NRHS > 0 && P == 16 && R == 2);
}

// NRHS = 0: potrf.  NRHS > 0: posv for up to NRHS right-hand sides (nrhs at
// run time), with the factor kept in registers for both triangular solves.
//
// PACKED (n = P R exactly, lda = n, stride = n*n, so a wavefront's G matrices
// are one contiguous run of memory): the referenced triangle is moved between
// HBM and registers through an LDS image of the wave's matrices, with
// consecutive lanes on consecutive elements, so every load and store
// instruction covers 64 consecutive elements.  Each element's (row, column,
// matrix) is tracked incrementally along the run; whether it is referenced is
// kept as one bit per element and lane, used again by the stores, so the other
// triangle is neither read nor written.  With n known at compile time, every
// LDS address of a row is a register plus an immediate offset.  The
// pivot-column exchange buffer reuses the image once the rows have been read
// out of it.  One wavefront per workgroup.  Otherwise each lane loads and
// stores its own rows (any order n <= P R, any layout).
template <typename T, int P, int R, bool UPPER, int NRHS, bool PACKED>
__global__ __launch_bounds__(PACKED ? 64 : 64 * kTinyWaves) void potrf_tiny_kernel(
    T* __restrict__ A, int n_arg, int64_t lda, int64_t stride, int64_t batch,
    int32_t* __restrict__ info, T* __restrict__ B, int nrhs, int64_t ldb, int64_t strideB,
    int gu)
{
    const int n = PACKED ? P * R : n_arg;
    using Rt = typename Traits<T>::R;
    constexpr int NB = P * R;
    constexpr int G = 64 / P;
    constexpr int PARTS = 63 / P + 1;     // includes a partial, dead tail partition
    constexpr int D = words<T>();
    constexpr int ROWW = tiny_row_words(NB + NRHS, D);
    constexpr int WAVES = PACKED ? 1 : kTinyWaves;
    constexpr int XW = 2 * PARTS * ROWW;                          // exchange words per wave
    constexpr int IMGW = PACKED ? packed_image_words<T, P, R>() : 0;
    constexpr bool SLABS = use_slabs<T, P, R, UPPER, NRHS, PACKED>();
    constexpr int SLABW = SLABS ? slab_tile_words<T>() : 0;
    constexpr int LDSW = cmax(cmax(XW, IMGW), SLABW);
    __shared__ __attribute__((aligned(16))) uint32_t lds_raw[WAVES][LDSW];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int p = lane / P;
    const int q = lane - p * P;
    const int GU = PACKED ? G : gu;       // matrices this wavefront takes (<= G; the rest idle)
    const int64_t b_first = ((int64_t)blockIdx.x * WAVES + wave) * GU;   // wave-uniform
    const int64_t b = b_first + p;
    const bool live = (p < GU) && (b < batch);
    uint32_t* const xbuf = &lds_raw[wave][0];
    auto xrow = [&](int par, int part) -> uint32_t* { return xbuf + (par * PARTS + part) * ROWW; };
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
    // packed path: element e of the wave's run is matrix ep, column ec, row ei
    constexpr int K = cdiv(G * NB * NB, 64);       // 64-element steps over the run
    constexpr int NBITS = cdiv(K, 32);
    constexpr int NN = NB * NB;
    constexpr int IMGP = packed_pitch<P, R>();
    uint32_t refbits[NBITS > 0 ? NBITS : 1];
    const int glive = int(batch - b_first < G ? batch - b_first : G);
    // masked offset: bit 31 puts a lane out of the buffer's range
    auto masked = [&](uint32_t o, bool ok) -> uint32_t { return o | (uint32_t(!ok) << 31); };
    // walks the run 64 elements at a time: element e = 64 v + lane is matrix
    // ep, column ec, row ei; calls f(v, e, image index, referenced)
    auto walk = [&](auto f, auto chunked) {
        // the lane index is hidden from the optimiser, so that the second walk
        // recomputes its offsets instead of keeping the first walk's live
        // across the factorisation
        int ln = lane;
        asm volatile("" : "+v"(ln));
        int ep = ln / NN;
        const int erem = ln - ep * NN;
        int ec = erem / NB;
        int ei = erem - ec * NB;
        constexpr int DI = 64 % NB, DQ = 64 / NB, DC = DQ % NB, DP = DQ / NB;
        static_for<0, K>([&](auto vv) {
            constexpr int v = vv;
            const int e = 64 * v + ln;
            const bool ok = ep < glive && (UPPER ? ei <= ec : ei >= ec);
            f(vv, e, e + ep * (IMGP - NN), ok);
            // the stores go out 16 at a time: otherwise every LDS read and
            // offset of the run is computed first and held in registers
            if constexpr (decltype(chunked)::value && v % 16 == 15) __builtin_amdgcn_sched_barrier(0);
            ei += DI;
            const bool ci = ei >= NB;
            ei = ci ? ei - NB : ei;
            ec += DC + (ci ? 1 : 0);
            const bool cc = ec >= NB;
            ec = cc ? ec - NB : ec;
            ep += DP + (cc ? 1 : 0);
        });
    };
    // image element of slot (r, c) of this lane's rows: element (i, c) of the
    // matrix for Lower, element (c, i) for Upper (i = q + r P)
    const int rowbase = UPPER ? p * IMGP + q * NB : p * IMGP + q;
    auto img_index = [&](int r, int c) -> int {
        return UPPER ? rowbase + (r * P) * NB + c : rowbase + r * P + c * NB;
    };
    if constexpr (PACKED) {
        static_for<0, NBITS>([&](auto ww) { refbits[ww] = 0u; });
        walk([&](auto vv, int e, int idx, bool ok) {
            constexpr int v = vv;
            refbits[v / 32] |= uint32_t(ok) << (v % 32);
            const T x = buf_load<T>(rsrc, masked(uint32_t(e) * S, ok));
            lds_put<T>(xbuf, idx, x);
        }, std::false_type{});
        wave_lds_sync();
    }
    if constexpr (SLABS) {
        constexpr int SR = slab_rows<T>(), CPI = 64 / SR, SPW = slab_pitch_words<T>();
        const int lr = lane % SR, lc = lane / SR;
        // every load first (element (sb SR + lr, u CPI + lc) of A; only the
        // referenced triangle of live columns is read, the rest comes back 0)
        T st[64 / SR][SR];
        static_for<0, 64 / SR>([&](auto sbc) {
            constexpr int sb = sbc;
            static_for<0, SR>([&](auto uc) {
                constexpr int u = uc;
                const int row = sb * SR + lr, col = u * CPI + lc;
                const bool ok = live && col < n && row <= col;
                st[sb][u] = buf_load<T>(rsrc, masked(uint32_t(col) * lda_b + uint32_t(row) * S, ok));
            });
        });
        // then slab by slab through the tile: lane i takes column i's SR rows
        static_for<0, 64 / SR>([&](auto sbc) {
            constexpr int sb = sbc;
            static_for<0, SR>([&](auto uc) {
                constexpr int u = uc;
                lds_put<T>(xbuf + (u * CPI + lc) * SPW, lr, st[sb][u]);
            });
            wave_lds_sync();
            static_for<0, SR>([&](auto rc) {
                constexpr int rr = rc;
                a[0][sb * SR + rr] = lds_get<T>(xbuf + lane * SPW, rr);
            });
            wave_lds_sync();
        });
    } else
    static_for<0, R>([&](auto rr) {
        constexpr int r = rr;
        const int i = q + r * P;
        static_for<0, cmin(NB, (r + 1) * P)>([&](auto cc) {
            constexpr int c = cc;
            T v;
            if constexpr (PACKED) {
                // rows of dead partitions read an unused image region; the
                // select below turns them (and padding) into the identity
                v = lds_get<T>(xbuf, img_index(r, c));
                v = select(live, v, zero<T>());
            } else {
                // Lower: the column offset goes in the scalar offset, so
                // each load needs no address register of its own
                uint32_t off = UPPER ? elem_off(r, c) : roff[r];
                if constexpr (c >= r * P) off = (c <= i) ? off : kBufOOB;   // diagonal block
                v = buf_load<T>(rsrc, off, UPPER ? 0u : uint32_t(c) * lda_b);
            }
            a[r][c] = v;
        });
    });
    // Every load is issued before the first use of a loaded value: otherwise
    // the scheduler may place each select right after its load and wait for
    // the loads one at a time.
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, R>([&](auto rr) {
        constexpr int r = rr;
        const int i = q + r * P;
        static_for<0, cmin(NB, (r + 1) * P)>([&](auto cc) {
            constexpr int c = cc;
            if constexpr (UPPER) a[r][c] = conj(a[r][c]);
            if constexpr (c >= r * P) a[r][c] = select(c == i && roff[r] == kBufOOB, one<T>(), a[r][c]);
        });
    });
    if constexpr (PACKED) wave_lds_sync();   // the exchange buffer reuses the image

    int32_t inf = 0;
    Rt invd[R];                 // 1 / L(i, i) of each held row (used by the solves)
    constexpr bool ONE_RSQ = one_rsq_window<T, P, R, NRHS>();
    if constexpr (P == 64 && R == 1)
        factor_rows_lane<T, UPPER, NRHS, ROWW, ONE_RSQ>(a, invd, xbuf, q, inf);
    else if constexpr (P == 16 && std::is_same<T, float>::value)
        factor_rows_dpp<T, R, UPPER, NRHS, ONE_RSQ>(a, invd, q, inf);
    else
        factor_rows<T, P, R, UPPER, NRHS, ROWW, ONE_RSQ>(a, invd, xbuf, p, q, inf);

    if constexpr (NRHS > 0)
        tiny_solves<T, P, R, NRHS>(a, invd, xbuf, PARTS * ROWW, ROWW, p, q, live, n,
                                   inf, B + b_first * strideB, nrhs, ldb, strideB);

    if constexpr (PACKED) {
        // rows back into the image (every lane writes; slots that are not
        // referenced elements go to the spare element), then the run back to HBM
        wave_lds_sync();
        // every slot is written back to its own image position: slots right of
        // the diagonal land on elements of the other triangle, which the run's
        // stores skip, and dead partitions write into their unused regions
        static_for<0, R>([&](auto rr) {
            constexpr int r = rr;
            static_for<0, cmin(NB, (r + 1) * P)>([&](auto cc) {
                constexpr int c = cc;
                lds_put<T>(xbuf, img_index(r, c), UPPER ? conj(a[r][c]) : a[r][c]);
            });
        });
        wave_lds_sync();
        walk([&](auto vv, int e, int idx, bool) {
            constexpr int v = vv;
            const bool ok = (refbits[v / 32] >> (v % 32)) & 1u;
            buf_store<T>(rsrc, masked(uint32_t(e) * S, ok), lds_get<T>(xbuf, idx));
        }, std::true_type{});
    } else if constexpr (SLABS) {
        // the loads in reverse: lane i puts column i's SR rows of the slab in
        // the tile, then each instruction stores whole lines of columns
        constexpr int SR = slab_rows<T>(), CPI = 64 / SR, SPW = slab_pitch_words<T>();
        int ln = lane;
        asm volatile("" : "+v"(ln));     // offsets recomputed here, not kept from the loads
        const int lr = ln % SR, lc = ln / SR;
        wave_lds_sync();
        static_for<0, 64 / SR>([&](auto sbc) {
            constexpr int sb = sbc;
            static_for<0, SR>([&](auto rc) {
                constexpr int rr = rc;
                lds_put<T>(xbuf + lane * SPW, rr, conj(a[0][sb * SR + rr]));
            });
            wave_lds_sync();
            static_for<0, SR>([&](auto uc) {
                constexpr int u = uc;
                const int row = sb * SR + lr, col = u * CPI + lc;
                const bool ok = live && col < n && row <= col;
                buf_store<T>(rsrc, masked(uint32_t(col) * lda_b + uint32_t(row) * S, ok),
                             lds_get<T>(xbuf + (u * CPI + lc) * SPW, lr));
            });
            wave_lds_sync();
        });
    } else {
        // With one matrix per wavefront the row fills most of the registers:
        // the row offset and index are hidden from the optimiser here, so that
        // the stores recompute their per-column offsets and masks instead of
        // keeping the loads' ones live across the factorisation (which leaves
        // the factor loop one staging register for its LDS reads).
        uint32_t roff_st[R];
        int q_st = q;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            roff_st[r] = roff[r];
            if constexpr (P == 64) asm volatile("" : "+v"(roff_st[r]));
        }
        if constexpr (P == 64) asm volatile("" : "+v"(q_st));
        static_for<0, R>([&](auto rr) {
            constexpr int r = rr;
            const int i = q_st + r * P;
            static_for<0, cmin(NB, (r + 1) * P)>([&](auto cc) {
                constexpr int c = cc;
                uint32_t off = UPPER ? roff_st[r] + uint32_t(c) * S : roff_st[r];
                if constexpr (c >= r * P) off = (c <= i) ? off : kBufOOB;
                if constexpr (UPPER) buf_store<T>(rsrc, off, conj(a[r][c]));
                else buf_store<T>(rsrc, off, a[r][c], uint32_t(c) * lda_b);
            });
        });
    }
    if (live && q == 0 && info != nullptr) info[b] = inf;
}

// ---------------------------------------------------------------- configurations
// P lanes x R rows per matrix; GU matrices per wavefront (at most 64 / P:
// fewer where measured faster, e.g. n = 33 takes 4 per wavefront, not 5).
template <int P_, int R_, int GU_ = 64 / P_> struct TC {
    static constexpr int P = P_, R = R_, NB = P_ * R_, GU = GU_;
    static_assert(GU_ >= 1 && GU_ <= 64 / P_, "matrices per wavefront");
};
template <typename... Cs> struct TList {};

// Ordered by order served (NB); the first entry with NB >= n is used.
template <typename T> struct TinyConfigs;
// (64 x 1: one matrix per wavefront, a lane per row, for orders 34..64; it
// needs more than 256 registers, so one wavefront per SIMD)
template <> struct TinyConfigs<float> {
    using type = TList<TC<4, 1>, TC<8, 1>, TC<6, 2>, TC<8, 2>, TC<17, 1>, TC<9, 2>, TC<8, 3>,
                       TC<16, 2>, TC<11, 3, 4>, TC<64, 1>>;
};
template <> struct TinyConfigs<double> {
    using type = TList<TC<4, 1>, TC<8, 1>, TC<6, 2>, TC<8, 2>, TC<8, 3>, TC<8, 4>, TC<64, 1>>;
};
template <> struct TinyConfigs<cfloat> {
    using type = TList<TC<4, 1>, TC<8, 1>, TC<6, 2>, TC<8, 2>, TC<8, 3>, TC<8, 4>, TC<64, 1>>;
};
template <> struct TinyConfigs<cdouble> {
    using type = TList<TC<4, 1>, TC<8, 1>, TC<6, 2>, TC<8, 2>, TC<32, 1>>;
};

// posv keeps more per lane (both solves' right-hand sides): smaller windows for
// the double types so that nothing spills.
template <typename T> struct PosvConfigs { using type = typename TinyConfigs<T>::type; };
template <> struct PosvConfigs<float> {
    using type = TList<TC<4, 1>, TC<8, 1>, TC<6, 2>, TC<8, 2>, TC<17, 1>, TC<9, 2>, TC<8, 3>,
                       TC<16, 2>, TC<11, 3>>;
};
template <> struct PosvConfigs<cfloat> {
    using type = TList<TC<4, 1>, TC<8, 1>, TC<6, 2>, TC<8, 2>, TC<8, 3>, TC<8, 4>>;
};
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

// The packed variant exists for fp32 (the element type of the bandwidth-bound
// workloads) and is used when n is the configuration's own order and the
// layout is packed.
template <typename T, typename C, bool UPPER>
constexpr bool packed_wanted() {
    return std::is_same<T, float>::value &&
           (UPPER ? packed_image_words<T, C::P, C::R>() * 4 <= kPackedUpperMaxBytes
                  : C::NB <= kPackedLowerMaxOrder);
}
template <typename C>
inline bool packed_layout(int n, int64_t lda, int64_t stride) {
    return n == C::NB && lda == n && stride == int64_t(n) * n;
}

template <typename T, typename List = typename TinyConfigs<T>::type>
bool geometry_t(bool upper, int n, int64_t lda, int64_t stride, int64_t batch, Geometry& g) {
    return pick_config(List{}, n, [&](auto c) {
        using C = decltype(c);
        constexpr int G = 64 / C::P;
        constexpr int D = words<T>();
        const bool packed = (upper ? packed_wanted<T, C, true>() : packed_wanted<T, C, false>()) &&
                            packed_layout<C>(n, lda, stride);
        const int waves = packed ? 1 : kTinyWaves;
        const int64_t xw = int64_t(2) * (63 / C::P + 1) * tiny_row_words(C::NB, D);
        const int64_t iw = packed_image_words<T, C::P, C::R>();
        g.family = FAM_TINY;
        g.P = C::P;
        g.R = C::R;
        const int gw = packed ? G : C::GU;      // matrices per wavefront
        g.G = gw;
        g.threads = 64 * waves;
        g.panel = 0;
        g.grid = (batch + gw * waves - 1) / (gw * waves);
        if (g.grid > kTinyMaxGrid) g.grid = kTinyMaxGrid;     // first launch of a sliced batch
        const int64_t sw = (upper && C::P == 64 && C::R == 1 && !packed) ? slab_tile_words<T>() : 0;
        g.lds = packed ? 4 * (xw > iw ? xw : iw) : int64_t(waves) * (xw > sw ? xw : sw) * 4;
    });
}

// One launch of the tiny kernel: the packed variant where the layout and the
// image size allow it, the per-row variant otherwise.
template <typename T, typename C, bool UPPER, int NRHS>
hipError_t launch_tiny(int n, T* a, int64_t lda, int64_t stride, int64_t batch, int32_t* info,
                       T* b, int nrhs, int64_t ldb, int64_t strideB, hipStream_t s) {
    constexpr int G = 64 / C::P;
    bool packed = false;
    if constexpr (packed_wanted<T, C, UPPER>()) packed = packed_layout<C>(n, lda, stride);
    const int gu = packed ? G : C::GU;                   // matrices per workgroup (one wavefront)
    const int64_t per_launch = kTinyMaxGrid * gu;        // matrices per launch
    hipError_t err = hipSuccess;
    for (int64_t b0 = 0; b0 < batch && err == hipSuccess; b0 += per_launch) {
        const int64_t nb = batch - b0 < per_launch ? batch - b0 : per_launch;
        const dim3 grid((unsigned)((nb + gu - 1) / gu));
        T* const as = a + b0 * stride;
        int32_t* const is = info ? info + b0 : nullptr;
        T* const bs = b ? b + b0 * strideB : nullptr;
        if (packed) {
            if constexpr (packed_wanted<T, C, UPPER>())
                err = launch(potrf_tiny_kernel<T, C::P, C::R, UPPER, NRHS, true>, grid, dim3(64), 0, s,
                             as, n, lda, stride, nb, is, bs, nrhs, ldb, strideB, gu);
        } else {
            err = launch(potrf_tiny_kernel<T, C::P, C::R, UPPER, NRHS, false>, grid,
                         dim3(64 * kTinyWaves), 0, s, as, n, lda, stride, nb, is, bs, nrhs, ldb,
                         strideB, gu);
        }
    }
    return err;
}

template <typename T>
hipError_t potrf_t(bool upper, int n, void* A, int64_t lda, int64_t stride, int64_t batch,
                   int32_t* info, hipStream_t s) {
    hipError_t err = hipErrorInvalidValue;
    pick_config(typename TinyConfigs<T>::type{}, n, [&](auto c) {
        using C = decltype(c);
        T* a = static_cast<T*>(A);
        T* nob = nullptr;
        if (upper)
            err = launch_tiny<T, C, true, 0>(n, a, lda, stride, batch, info, nob, 0, 0, 0, s);
        else
            err = launch_tiny<T, C, false, 0>(n, a, lda, stride, batch, info, nob, 0, 0, 0, s);
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
        T* a = static_cast<T*>(A);
        T* bb = static_cast<T*>(B);
        if (nrhs == 1) {
            if (upper) err = launch_tiny<T, C, true, 1>(n, a, lda, strideA, batch, info, bb, nrhs, ldb, strideB, s);
            else err = launch_tiny<T, C, false, 1>(n, a, lda, strideA, batch, info, bb, nrhs, ldb, strideB, s);
        } else {
            if (upper) err = launch_tiny<T, C, true, kPosvMaxRhs>(n, a, lda, strideA, batch, info, bb, nrhs, ldb, strideB, s);
            else err = launch_tiny<T, C, false, kPosvMaxRhs>(n, a, lda, strideA, batch, info, bb, nrhs, ldb, strideB, s);
        }
    });
    return err;
}

}  // namespace tiny_detail
}  // namespace bl
