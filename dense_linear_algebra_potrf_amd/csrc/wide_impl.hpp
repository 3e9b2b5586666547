// Wide window of the tiny family (implementation header): orders up to 192
// above the one-wavefront windows (from 65; from 33 for complex double), one
// workgroup per matrix, the matrix held in the registers of several wavefronts.
//
// Prior art: the BatchLAS perf_potrf page, section "potrf: the tiny tier"
// (lane r owns row r and every value stays in registers) and section "The
// LPanel tier" (one thread per row at mid orders).  Beyond 64 rows one
// wavefront no longer holds a row per lane, and two rows per lane do not fit
// the register file at a useful occupancy, so the rows are spread over the
// wavefronts of a workgroup.  Two layouts:
//
//   * rows (fp32, orders 65..128): two wavefronts, lane l of wavefront w holding
//     row 64 w + l whole.  A row only has columns up to its diagonal, so wavefront
//     w keeps the columns below 64 (w + 1), fixed at compile time for each
//     wavefront's code: wavefront 0 stops updating after column 63.
//   * tiles (fp32 orders 129..192, the other types throughout, where a whole
//     row per lane would need 2n registers or more): the part below the diagonal cut
//     into tiles of 64 rows x 32 columns, one wavefront per tile (up to 12);
//     lane l of the wavefront for row block rb and column block cb holds
//     columns 32 cb .. 32 cb + 31 of row 64 rb + l.
//
// The column recurrence is that of the tiny family (right-looking, the Schur
// pivot never stale, the multiplier s_ij / d applied to the unscaled column,
// failures as selects with the first failing column kept).  Column j is
// exchanged through an LDS buffer with one slot per row, double-buffered by
// step parity; one workgroup barrier ends each step, which orders each column's
// stores before its reads and the reads of a buffer before its reuse two steps
// later.  The entries of column j a row's update needs lie in groups of 16
// rows: lane q reads entry 16 g + (q mod 16) of group g, and each update takes
// its row's value from the right lane of its row of 16 by a DPP broadcast
// inside the multiply-add, so one LDS read per lane feeds 16 updates.  Complex
// elements follow the tiny family: the pivot is the real part of the diagonal,
// the update is s_ik -= (s_ij / d) conj(s_kj), and Upper works on
// S = conj(A^T).
//
// Loads and stores (Lower): lanes of a wavefront hold consecutive rows, so
// each column is one coalesced access of 64 consecutive elements.  Upper reads
// S(i, c) = A(c, i): the tiles layout a row of A per lane, the rows layout in
// slabs of whole column lines through an LDS tile.
#pragma once

#include "families.hpp"

namespace bl {
namespace wide_detail {

constexpr int kWideRowsMaxOrder = 128;           // the rows layout serves fp32 65..128
constexpr int kWideMaxOrder = 192;               // the tiles layout the rest, to 192
constexpr int kTileCols = 32;                    // columns of a tile
constexpr int kWideSlots = kWideMaxOrder + 4;    // slots of each column buffer
constexpr int64_t kWideMaxGrid = int64_t(1) << 20;

// One matrix's buffer descriptor and the byte offsets of its elements.
template <typename T>
struct WideRow {
    __amdgpu_buffer_rsrc_t rs;
    uint32_t lda_b;
    // Column c's scalar offset, computed next to its use behind an opaque copy:
    // otherwise all of them are computed once, hoisted out of the batch loop
    // and held (spilled) for the whole factorisation.
    template <bool UPPER>
    __device__ __forceinline__ uint32_t col_off(int c) const {
        uint32_t step = UPPER ? uint32_t(sizeof(T)) : lda_b;
        asm volatile("" : "+s"(step) : : "memory");
        return uint32_t(c) * step;
    }
    // Row i's offset for its element of column c, or out of range for rows at
    // or beyond n and for entries above the diagonal.
    template <bool UPPER>
    __device__ __forceinline__ uint32_t off(int i, int c, int n) const {
        return (c <= i && i < n) ? (UPPER ? uint32_t(i) * lda_b : uint32_t(i) * uint32_t(sizeof(T)))
                                 : kBufOOB;
    }
};

// The row index behind an opaque copy.  Everything derived from the row index
// (masked offsets, the diagonal select) is formed from a fresh copy where it is
// used: shared between the loads and the stores, or hoisted out of the batch
// loop, those values would be held (and spilled) across the factorisation.
__device__ __forceinline__ int opaque_row(int i) {
    asm volatile("" : "+v"(i));
    return i;
}

// The multiplier of a step, as the update's multiply-adds take it: -t for the
// real types; for the complex ones acc -= t conj(c) is
//   acc.re += (-t.re) c.re + (-t.im) c.im,   acc.im += (-t.im) c.re + t.re c.im.
template <typename T> struct WideMult { T n; };
template <> struct WideMult<cfloat> { float nre, nim, tre; };
template <> struct WideMult<cdouble> { double nre, nim, tre; };
template <typename T>
__device__ __forceinline__ WideMult<T> wide_mult(const T& t) {
    if constexpr (Traits<T>::cplx) return WideMult<T>{-t.re, -t.im, t.re};
    else return WideMult<T>{-t};
}

// acc -= t conj(x), x taken from lane N of this lane's row of 16
template <int N, bool FIRST, typename T>
__device__ __forceinline__ void wide_fma16(T& acc, const WideMult<T>& m, const T& col) {
    if constexpr (Traits<T>::cplx) {
        fma_bcast16<N, FIRST>(acc.re, m.nre, col.re);
        fma_bcast16<N, false>(acc.re, m.nim, col.im);
        fma_bcast16<N, false>(acc.im, m.nim, col.re);
        fma_bcast16<N, false>(acc.im, m.tre, col.im);
    } else {
        fma_bcast16<N, FIRST>(acc, m.n, col);
    }
}

// Rank-1 update of a[K0..KE) with multiplier m against the column entries
// col[c0 + k], in groups of 16 rows with DPP row broadcasts.
template <int K0, int KE, typename T, int N>
__device__ __forceinline__ void wide_update(T (&a)[N], const T* col, int c0, int q16, const WideMult<T>& m) {
    if constexpr (K0 < KE) {
        constexpr int G0 = K0 / 16, G1 = (KE + 15) / 16;
        T cg[2];
        cg[G0 & 1] = col[c0 + 16 * G0 + q16];
        static_for<G0, G1>([&](auto gg) {
            constexpr int g = gg;
            if constexpr (g + 1 < G1) cg[(g + 1) & 1] = col[c0 + 16 * (g + 1) + q16];
            constexpr int KB = cmax(K0, 16 * g);
            static_for<KB, cmin(KE, 16 * g + 16)>([&](auto kk) {
                constexpr int k = kk;
                wide_fma16<k - 16 * g, k == KB>(a[k], m, cg[g & 1]);
            });
        });
    }
}

// info: the first failing pivot (1-based), kept once set
template <typename R>
__device__ __forceinline__ void note_pivot(int32_t& inf, R d, int j) {
    inf = (inf == 0 && !(d > R(0))) ? (j + 1) : inf;
    // taken now: sunk into the final store, the select chain would keep every
    // pivot alive across the factorisation
    asm volatile("" : "+v"(inf));
}

// ---------------------------------------------------------------- rows layout
// NC = 96 or 128 columns (two wavefronts; rows beyond 96 are idle for n <= 96).
template <int NC, bool UPPER>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(3))) void potrf_wide_rows_kernel(
    float* __restrict__ A, int n, int64_t lda, int64_t stride, int64_t batch,
    int32_t* __restrict__ info)
{
    __shared__ __attribute__((aligned(16))) float colbuf[2][kWideSlots];
    // Upper: lane i's row is column i of A, so loads and stores per row would
    // touch a cache line per lane and element.  The referenced triangle moves
    // instead in slabs of 32 rows of A (one 128-byte line of every column):
    // each instruction of the workgroup covers four whole column lines, and a
    // tile of 32 elements (plus one of padding) for each of the workgroup's
    // 128 rows transposes the slab (rows beyond NC are idle: they read what
    // the tile holds and write their own slots, which no one reads).  Each
    // final column of the factor goes into the tile at its step; every 32
    // steps the slab is written out as whole lines.
    constexpr int SR = 32, PITCH = SR + 1;
    __shared__ __attribute__((aligned(16))) float tile[UPPER ? 128 * PITCH : 1];
    const int lane = threadIdx.x & 63;
    const int q16 = lane & 15;                // lane within its row of 16 (DPP broadcasts)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = wave * 64 + lane;           // this lane's row
    const int lr = threadIdx.x & 31, lc = threadIdx.x >> 5;   // slab: row of A, column within 4

    // the whole matrix for the wavefront whose rows end at KE
    auto run = [&](auto kec, int64_t b) __attribute__((always_inline)) {
        constexpr int KE = decltype(kec)::value;
        const WideRow<float> m{make_rsrc(A + b * stride), uint32_t(lda) * 4u};
        // Rows at or beyond n load as zero and are never stored; a row's update
        // only reads the column entries of rows at or above it, so their values
        // never reach a row below n.  Their first zero pivot (step n) only marks
        // info n + 1, which is cleared at the end.
        // Upper, slabs: element (row r, column c) of A, out of range unless
        // r <= c < n (row and column behind opaque copies at every use)
        auto slab_off = [&](int c, int r) __attribute__((always_inline)) {
            c = opaque_row(c);
            r = opaque_row(r);
            return (r <= c && c < n) ? uint32_t(c) * m.lda_b + uint32_t(r) * 4u : kBufOOB;
        };
        float a[KE];
        if constexpr (!UPPER) {
            const int il = opaque_row(i);
            static_for<0, KE>([&](auto cc) {
                constexpr int c = cc;
                a[c] = buf_load<float>(m.rs, m.off<UPPER>(il, c, n), m.col_off<UPPER>(c));
            });
        } else {
            // slab sb: rows 32 sb .. 32 sb + 31 of A in the columns that reach
            // them (>= 32 sb); entries right of a row's diagonal are left as
            // they come (never stored, never read by a referenced entry)
            static_for<0, NC / SR>([&](auto sbc) {
                constexpr int sb = sbc, U0 = sb * SR / 4, NU = NC / 4;
                float st[NU - U0];
                static_for<U0, NU>([&](auto uc) {
                    constexpr int u = uc;
                    st[u - U0] = buf_load<float>(m.rs, slab_off(u * 4 + lc, sb * SR + lr));
                });
                float* tw = tile + opaque_row(lc * PITCH + lr);
                static_for<U0, NU>([&](auto uc) {
                    constexpr int u = uc;
                    tw[u * 4 * PITCH] = st[u - U0];
                });
                __syncthreads();
                const float* tr = tile + opaque_row(i * PITCH);
                static_for<0, SR>([&](auto rc) {
                    constexpr int c = sb * SR + rc;
                    if constexpr (c < KE) a[c] = tr[rc];
                });
                __syncthreads();
            });
        }
        int32_t inf = 0;
        colbuf[0][i] = a[0];
        __syncthreads();
        static_for<0, NC>([&](auto jj) {
            constexpr int j = jj;
            if constexpr (j < KE) {
                const float* col = &colbuf[j & 1][0];
                const float d = col[j];
                note_pivot(inf, d, j);
                float inv, rsd, sq;
                pivot_terms(d, inv, rsd, sq);
                const float t = a[j] * inv;
                // the next column first, published for the next step
                if constexpr (j + 1 < KE) {
                    a[j + 1] = fmadd(-t, col[j + 1], a[j + 1]);
                    colbuf[(j + 1) & 1][i] = a[j + 1];
                }
                wide_update<j + 2, KE>(a, col, 0, q16, WideMult<float>{-t});
                // column j is final: to the matrix now (Lower: one coalesced
                // column; Upper: into the tile), which frees its register for
                // the rest of the factorisation
                const int is = opaque_row(i);
                const float lij = (is == j) ? sq : a[j] * rsd;
                if constexpr (UPPER) tile[is * PITCH + j % SR] = lij;
                else buf_store<float>(m.rs, m.off<UPPER>(is, j, n), lij, m.col_off<UPPER>(j));
            }
            __syncthreads();
            if constexpr (UPPER && j % SR == SR - 1) {
                // slab j / 32 of the factor, as whole lines of A (every thread)
                constexpr int sb = j / SR, U0 = sb * SR / 4, NU = NC / 4;
                const float* tr = tile + opaque_row(lc * PITCH + lr);
                static_for<U0, NU>([&](auto uc) {
                    constexpr int u = uc;
                    buf_store<float>(m.rs, slab_off(u * 4 + lc, sb * SR + lr), tr[u * 4 * PITCH]);
                });
                __syncthreads();
            }
        });
        // the second wavefront reads every pivot (the first stops at its last row)
        if (wave == 1 && lane == 0 && info != nullptr) info[b] = inf > n ? 0 : inf;
    };

    for (int64_t b = blockIdx.x; b < batch; b += gridDim.x) {
        if (wave == 0) run(ic<64>{}, b);
        else run(ic<NC>{}, b);
        __syncthreads();     // colbuf is reused by the next matrix
    }
}

// ---------------------------------------------------------------- tiles layout
// Row block rb holds the column blocks that start below min(64 (rb + 1), n);
// wavefronts are numbered row block by row block.
__host__ __device__ constexpr int wide_col_blocks(int rb, int n) {
    return ((64 * (rb + 1) < n ? 64 * (rb + 1) : n) + kTileCols - 1) / kTileCols;
}
__host__ __device__ constexpr int wide_tile_waves(int n) {
    int w = 0;
    for (int rb = 0; 64 * rb < n; ++rb) w += wide_col_blocks(rb, n);
    return w;
}
static_assert(wide_tile_waves(kWideMaxOrder) <= 12, "the tiles layout fits 768 threads");

// A wavefront's steps fall in three phases:
//   * before its tile's block (j < c0): every entry of the tile takes the
//     rank-1 update, the multiplier read from the slot of its own row;
//   * inside it: the recurrence on the tile's triangle, unrolled at compile time
//     relative to the block, publishing the next column of its rows and storing
//     the finished one at every step;
//   * after it: barriers only.
// Every wavefront runs the same code, its tile decided at run time, so one
// kernel serves every order.
template <typename T, bool UPPER>
__global__ __launch_bounds__(768) void potrf_wide_tiles_kernel(T* __restrict__ A, int n, int64_t lda,
                                                               int64_t stride, int64_t batch,
                                                               int32_t* __restrict__ info)
{
    using R = typename Traits<T>::R;
    constexpr int CB = kTileCols;
    __shared__ __attribute__((aligned(16))) T colbuf[2][kWideSlots];

    const int lane = threadIdx.x & 63;
    const int q16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int rb = 0, cb = wave;
    while (cb >= wide_col_blocks(rb, n)) {
        cb -= wide_col_blocks(rb, n);
        ++rb;
    }
    const int c0 = cb * CB;                   // first column of the tile
    const int nstep = (n + CB - 1) / CB * CB; // steps run by every wavefront
    const bool reports = wave == wide_tile_waves(n) - 1;   // sees every pivot below n
    const int i = rb * 64 + lane;

    for (int64_t b = blockIdx.x; b < batch; b += gridDim.x) {
        const WideRow<T> m{make_rsrc(A + b * stride), uint32_t(lda) * uint32_t(sizeof(T))};
        // Rows at or beyond n load as zero and are never stored, and cannot
        // reach a row below n (as in the rows layout).  Upper holds
        // S(i, c) = conj(A(c, i)): conjugated on the way in and out.
        T a[CB];
        const int il = opaque_row(i);
        static_for<0, CB>([&](auto cc) {
            constexpr int c = cc;
            const T v = buf_load<T>(m.rs, m.template off<UPPER>(il, c0 + c, n), m.template col_off<UPPER>(c0 + c));
            a[c] = UPPER ? conj(v) : v;
        });
        int32_t inf = 0;
        if (c0 == 0) colbuf[0][i] = a[0];
        __syncthreads();

        // before the tile's block: the whole tile takes every step's update
        for (int j = 0; j < c0; ++j) {
            const T* col = colbuf[j & 1];
            const R d = re(col[j]);
            note_pivot(inf, d, j);
            wide_update<0, CB>(a, col, c0, q16, wide_mult(scale(col[i], pivot_rcp(d))));
            if (j + 1 == c0) colbuf[(j + 1) & 1][i] = a[0];
            __syncthreads();
        }
        // inside it: the triangle, relative to the block (c0 is even, so the
        // parity of column c0 + jj is that of jj)
        static_for<0, CB>([&](auto jc) {
            constexpr int jj = jc;
            const int j = c0 + jj;
            const T* col = colbuf[jj & 1];
            const R d = re(col[j]);
            note_pivot(inf, d, j);
            R inv, rsd, sq;
            pivot_terms(d, inv, rsd, sq);
            if constexpr (jj + 1 < CB) {
                wide_update<jj + 1, CB>(a, col, c0, q16, wide_mult(scale(a[jj], inv)));
                colbuf[(jj + 1) & 1][i] = a[jj + 1];
            }
            const int is = opaque_row(i);
            const T lij = select(is == j, diag_value<T>(sq, UPPER), scale(a[jj], rsd));
            buf_store<T>(m.rs, m.template off<UPPER>(is, j, n), UPPER ? conj(lij) : lij,
                         m.template col_off<UPPER>(j));
            __syncthreads();
        });
        // after it: keep step with the other wavefronts
        for (int j = c0 + CB; j < nstep; ++j) __syncthreads();

        if (reports && lane == 0 && info != nullptr) info[b] = inf > n ? 0 : inf;
        __syncthreads();     // colbuf is reused by the next matrix
    }
}

// ---------------------------------------------------------------- host side
// Orders served: above the one-wavefront windows.
constexpr int kWideMinOrder = 65;

// The rows layout is used for fp32 up to order 128, the tiles layout otherwise.
template <typename T>
inline bool wide_rows(int n) { return std::is_same<T, float>::value && n <= kWideRowsMaxOrder; }

// Every offset inside one matrix (at most (n - 1)(lda + 1) elements, which the
// stride bounds) must fit the 31-bit buffer offsets.
template <typename T>
inline bool wide_layout_ok(int64_t stride) { return stride <= int64_t(0x7fffffff) / int64_t(sizeof(T)); }

template <typename T>
inline int wide_threads(int n) { return wide_rows<T>(n) ? 128 : 64 * wide_tile_waves(n); }

template <typename T>
inline void wide_geometry(bool upper, int n, int64_t batch, Geometry& g) {
    g.family = FAM_TINY;
    g.threads = wide_threads<T>(n);
    g.P = g.threads;                                         // lanes sharing one matrix
    g.R = 1;
    g.G = 1;                                                 // one matrix per workgroup
    g.panel = wide_rows<T>(n) ? 0 : kTileCols;               // columns of a tile
    g.grid = batch < kWideMaxGrid ? batch : kWideMaxGrid;
    g.lds = int64_t(2) * kWideSlots * int64_t(sizeof(T));
    if (upper && wide_rows<T>(n)) g.lds += int64_t(128) * 33 * 4;   // the slab tile
}

// Enqueue one element type and triangle (instantiated by its translation unit).
template <typename T, bool UPPER>
hipError_t wide_launch(int n, T* a, int64_t lda, int64_t stride, int64_t batch, int32_t* info,
                       hipStream_t s) {
    const dim3 gd((unsigned)(batch < kWideMaxGrid ? batch : kWideMaxGrid));
    const dim3 bd(wide_threads<T>(n));
    if constexpr (std::is_same<T, float>::value) {
        if (n <= 96)
            return launch(potrf_wide_rows_kernel<96, UPPER>, gd, bd, 0, s, a, n, lda, stride, batch, info);
        if (n <= kWideRowsMaxOrder)
            return launch(potrf_wide_rows_kernel<128, UPPER>, gd, bd, 0, s, a, n, lda, stride, batch, info);
    }
    return launch(potrf_wide_tiles_kernel<T, UPPER>, gd, bd, 0, s, a, n, lda, stride, batch, info);
}

}  // namespace wide_detail
}  // namespace bl
