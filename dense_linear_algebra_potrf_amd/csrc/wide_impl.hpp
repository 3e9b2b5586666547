// Wide window of the tiny family (implementation header): orders 65..128 in
// fp32, one workgroup of two wavefronts per matrix, each lane holding one row
// of the matrix in registers.
//
// Prior art: the BatchLAS perf_potrf page, section "potrf: the tiny tier"
// (lane r owns row r and every value stays in registers) and section "The
// LPanel tier" (one thread per row at mid orders).  Beyond 64 rows one
// wavefront no longer holds a row per lane, and two rows per lane do not fit
// the register file at a useful occupancy, so the rows are split over the
// wavefronts of a workgroup: wavefront w holds rows 64 w .. 64 w + 63, lane l
// row 64 w + l.  A row only has columns up to its diagonal, so wavefront w
// keeps the columns below KE(w) = 64 (w + 1) (fixed at compile time for each
// wavefront's code); wavefront 0 stops updating after column 63.
//
// The column recurrence is that of the tiny family (right-looking, the
// Schur pivot never stale, the multiplier s_ij / d applied to the unscaled
// column, failures as selects with the first failing column kept), with the
// pivot column exchanged through LDS between the wavefronts: at step j every
// lane has the entries of column j it needs in the buffer of parity j; it
// updates its entry of column j + 1 first and publishes it to the other
// buffer, then the rest of its row, and one workgroup barrier ends the step.
// The barrier separates each column's stores from its reads, and the reads of
// a buffer from its reuse two steps later.
//
// Loads and stores (Lower): lanes of a wavefront hold consecutive rows, so
// each column is one coalesced access of 64 consecutive elements.  Upper reads
// S(i, c) = A(c, i), a row of A per lane.
#pragma once

#include "families.hpp"

namespace bl {
namespace wide_detail {

// Columns (and rows) served: NC = 96 or 128; two wavefronts per workgroup.
template <int NC> struct WideShape {
    static constexpr int NW = (NC + 63) / 64;
    static constexpr int LD = 64 * NW + 4;   // floats per column buffer: a slot for every lane
};

constexpr int64_t kWideMaxGrid = int64_t(1) << 20;

template <int NC, bool UPPER, bool ONE_RSQ>
__global__ __launch_bounds__(64 * WideShape<NC>::NW) __attribute__((amdgpu_waves_per_eu(2))) void potrf_wide_kernel(
    float* __restrict__ A, int n, int64_t lda, int64_t stride, int64_t batch,
    int32_t* __restrict__ info)
{
    using Sh = WideShape<NC>;
    constexpr int NW = Sh::NW, LD = Sh::LD;
    __shared__ __attribute__((aligned(16))) float colbuf[2][LD];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i0 = wave * 64 + lane;          // this lane's row
    const uint32_t lda_b = uint32_t(lda) * 4u;

    // the whole matrix for the wavefront whose rows end at KE
    auto run = [&](auto kec, int64_t b) __attribute__((always_inline)) {
        constexpr int KE = decltype(kec)::value;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(A + b * stride);
        // the row index hidden from the optimiser: the masked offsets are the
        // same for every matrix, and hoisted out of the batch loop they would
        // be held in registers across the factorisation
        int i = i0;
        asm volatile("" : "+v"(i));
        const bool rowok = i < n;
        const uint32_t rbase = rowok ? (UPPER ? uint32_t(i) * lda_b : uint32_t(i) * 4u) : kBufOOB;
        // Column c's scalar offset is computed next to its use, behind an opaque
        // copy: otherwise all of them are computed once, hoisted out of the batch
        // loop and held (spilled) for the whole factorisation.
        auto col_off = [&](int c) __attribute__((always_inline)) {
            uint32_t step = UPPER ? 4u : lda_b;
            asm volatile("" : "+s"(step) : : "memory");
            return uint32_t(c) * step;
        };
        float a[KE];
        static_for<0, KE>([&](auto cc) {
            constexpr int c = cc;
            // the diagonal block's upper part is never read (scratch slots)
            uint32_t off = rbase;
            if constexpr (c >= KE - 64) off = (c <= i) ? off : kBufOOB;
            a[c] = buf_load<float>(rs, off, col_off(c));
        });
        // Rows at or beyond n load as zero and are never stored (rbase is out of
        // range for them); a row's update only reads the column entries of rows
        // at or above it, so their values never reach a row below n.  Their first
        // zero pivot (step n) only marks info n + 1, which is cleared at the end.
        int32_t inf = 0;
        colbuf[0][i] = a[0];
        __syncthreads();
        static_for<0, NC>([&](auto jj) {
            constexpr int j = jj;
            if constexpr (j < KE) {
                const float* col = &colbuf[j & 1][0];
                const float d = col[j];
                inf = (inf == 0 && !(d > 0.0f)) ? (j + 1) : inf;
                // taken now: sunk into the store at the end, the select chain
                // would keep every pivot alive across the factorisation
                asm volatile("" : "+v"(inf));
                float inv, rsd, sq;
                if constexpr (ONE_RSQ) {
                    pivot_terms(d, inv, rsd, sq);
                } else {
                    inv = pivot_rcp(d);
                    rsd = pivot_rsq(d);
                    sq = pivot_sqrt(d);
                }
                const float t = a[j] * inv;
                if constexpr (j + 1 < KE) {
                    a[j + 1] = fmadd(-t, col[j + 1], a[j + 1]);
                    colbuf[(j + 1) & 1][i] = a[j + 1];
                }
                // the rest of the row, 16 columns a batch with the next batch's
                // reads issued ahead of this batch's updates
                constexpr int K0 = j + 2, CH = 16;
                if constexpr (K0 < KE) {
                    constexpr int NCH = (KE - K0 + CH - 1) / CH;
                    float cv[2][CH];
                    auto fetch = [&](auto ch) {
                        constexpr int c = ch;
                        static_for<K0 + c * CH, cmin(KE, K0 + (c + 1) * CH)>([&](auto kk) {
                            constexpr int k = kk;
                            cv[c & 1][k - K0 - c * CH] = col[k];
                        });
                    };
                    auto apply = [&](auto ch) {
                        constexpr int c = ch;
                        static_for<K0 + c * CH, cmin(KE, K0 + (c + 1) * CH)>([&](auto kk) {
                            constexpr int k = kk;
                            a[k] = fmadd(-t, cv[c & 1][k - K0 - c * CH], a[k]);
                        });
                    };
                    fetch(ic<0>{});
                    static_for<0, NCH>([&](auto ch) {
                        constexpr int c = ch;
                        __builtin_amdgcn_sched_barrier(0);
                        if constexpr (c + 1 < NCH) fetch(ic<c + 1>{});
                        apply(ch);
                    });
                    __builtin_amdgcn_sched_barrier(0);
                }
                // column j is final: to the matrix now (one coalesced column),
                // which frees its register for the rest of the factorisation
                const float lij = (i == j) ? sq : a[j] * rsd;
                buf_store<float>(rs, (j <= i) ? rbase : kBufOOB, lij, col_off(j));
            }
            __syncthreads();
        });
        // the last wavefront reads every pivot (the others stop at their last row)
        if (wave == NW - 1 && lane == 0 && info != nullptr) info[b] = inf > n ? 0 : inf;
    };

    for (int64_t b = blockIdx.x; b < batch; b += gridDim.x) {
        if (NW == 1 || wave == 0) run(ic<64>{}, b);
        else run(ic<NC>{}, b);
        __syncthreads();     // colbuf is reused by the next matrix
    }
}

// Orders served (fp32): above the one-wavefront windows, up to two wavefronts.
constexpr int kWideMinOrder = 65, kWideMaxOrder = 128;

// Every offset inside one matrix (at most (n - 1)(lda + 1) elements, which the
// stride bounds) must fit the 31-bit buffer offsets.
inline bool wide_layout_ok(int64_t stride) { return stride <= int64_t(0x7fffffff) / 4; }

// The window (96 or 128 columns) that serves order n.
inline int wide_window(int n) { return n <= 96 ? 96 : 128; }

inline void wide_geometry(int n, int64_t batch, Geometry& g) {
    g.family = FAM_TINY;
    g.P = 64 * ((wide_window(n) + 63) / 64);   // lanes holding one matrix (a row each)
    g.R = 1;
    g.G = 1;                                    // one matrix per workgroup
    g.threads = g.P;
    g.panel = 0;
    g.grid = batch < kWideMaxGrid ? batch : kWideMaxGrid;
    g.lds = int64_t(2) * (wide_window(n) == 96 ? WideShape<96>::LD : WideShape<128>::LD) * 4;
}

// Enqueue both windows of one triangle (instantiated by the translation unit
// of that triangle).
template <bool UPPER>
hipError_t wide_launch(int n, float* a, int64_t lda, int64_t stride, int64_t batch, int32_t* info,
                       hipStream_t s) {
    const dim3 gd((unsigned)(batch < kWideMaxGrid ? batch : kWideMaxGrid));
    if (wide_window(n) == 96)
        return launch(potrf_wide_kernel<96, UPPER, true>, gd, dim3(64 * WideShape<96>::NW), 0, s, a,
                      n, lda, stride, batch, info);
    return launch(potrf_wide_kernel<128, UPPER, true>, gd, dim3(64 * WideShape<128>::NW), 0, s, a,
                  n, lda, stride, batch, info);
}

}  // namespace wide_detail
}  // namespace bl
