// Folded window of the tiny family (implementation header): orders 33..64, two
// matrices per wavefront, 32 lanes per matrix, lane q holding rows q and 63 - q.
//
// Prior art: the BatchLAS perf_potrf page, section "potrf: the tiny tier" (lane
// r owns row r, every value in registers).  With one row per lane (the 64 x 1
// window) every lane of the wavefront updates every column right of the pivot,
// while row i only has columns up to i: half of the updates land in scratch
// slots.  Folding the rows pairs a short row with a long one: row q (q < 32)
// keeps columns 0..31 and row 63 - q columns 0..63, so at step j a lane updates
// (31 - j) + (63 - j) entries for two rows where the 64 x 1 window updates
// 63 - j for one, about a third fewer updates per matrix, and each entry of
// the pivot column read from LDS serves both of the lane's rows.  The
// recurrence is the tiny family's (right-looking, the Schur pivot never stale,
// the multiplier s_ij / d on the unscaled column, failures as selects); the
// pivot column goes through LDS, double-buffered by step parity, one buffer
// per matrix (per half-wavefront), with no barrier inside the wavefront.
// Rows at or beyond n hold the identity, so the steps past n see d = 1.
#pragma once

#include "families.hpp"

namespace bl {
namespace fold_detail {

constexpr int kFoldMin = 33, kFoldMax = 64;
constexpr int64_t kFoldMaxGrid = int64_t(1) << 19;     // workgroups of one wavefront (two matrices)

// An opaque copy: the column and row indices of the slab passes are shared by
// the loads and the stores; formed once, all of them would be held across the
// factorisation.
__device__ __forceinline__ int opaque_v(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

template <typename T, bool UPPER>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void potrf_fold_kernel(
    T* __restrict__ A, int n, int64_t lda, int64_t stride, int64_t batch, int32_t* __restrict__ info)
{
    using R = typename Traits<T>::R;
    constexpr uint32_t S = sizeof(T);
    // Upper: lane q's rows are columns q and 63 - q of A, so loads and stores
    // per row would touch a cache line per lane and element.  The referenced
    // triangle instead moves in slabs of SR rows of A (SR elements = one
    // 128-byte line of a column): each instruction covers whole lines (LPI
    // columns per matrix), the slab is transposed through a tile of 64
    // columns per matrix (a column's SR elements plus one element of
    // padding), and every lane picks its two columns out of it.  A slab of the
    // factor is written as soon as its SR columns are final.  (Only types of
    // up to 8 bytes: 192 values per lane.)
    static_assert(S <= 8, "two rows of 96 entries per lane");
    constexpr int SR = 128 / int(S), LPI = 32 / SR, PITCH = SR + 1;
    constexpr int CB = 2 * 2 * (64 + 4), TILE = UPPER ? 2 * 64 * PITCH : 0;
    __shared__ __attribute__((aligned(16))) T lds[CB + TILE];
    auto colbuf = [&](int par, int mh) __attribute__((always_inline)) { return lds + (par * 2 + mh) * (64 + 4); };

    const int lane = threadIdx.x & 63;
    const int h = lane >> 5;                  // which of the two matrices
    const int q = lane & 31;
    const uint32_t lda_b = uint32_t(lda) * S;

    for (int64_t m0 = 2 * int64_t(blockIdx.x); m0 < batch; m0 += 2 * int64_t(gridDim.x)) {
        const int64_t mat = m0 + h;
        const bool live = mat < batch;
        // one descriptor for the pair (a descriptor must be the same for the
        // whole wavefront), the second matrix at a byte offset inside it
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(A + m0 * stride);
        const uint32_t mbase = h ? uint32_t(stride) * S : 0u;
        // row `row`'s element of column c (out of range: masked), behind an
        // opaque copy of the row so that nothing derived from it is held
        // across the factorisation
        auto off = [&](int row, int c) __attribute__((always_inline)) {
            asm volatile("" : "+v"(row));
            uint32_t ldb = lda_b;            // (the column offsets are formed where used)
            asm volatile("" : "+s"(ldb));
            int lim = live ? n : 0;          // a missing second matrix has no rows
            asm volatile("" : "+v"(lim));
            uint32_t mb = mbase;             // (else mbase + c S is held for every c)
            asm volatile("" : "+v"(mb));
            const bool ok = (row < lim) & (c <= row);
            return ok ? mb + (UPPER ? uint32_t(row) * ldb + uint32_t(c) * S
                                       : uint32_t(c) * ldb + uint32_t(row) * S)
                      : kBufOOB;
        };
        // rows at or beyond n: the identity (n behind an opaque copy: the
        // comparisons with every column are otherwise hoisted and held)
        auto ident = [&](int row, int c, const T& v) __attribute__((always_inline)) {
            int r2 = row, nn = n;
            asm volatile("" : "+v"(r2), "+s"(nn));
            return (r2 >= nn && c == r2) ? one<T>() : v;
        };
        T xa[32], xb[64];
        const int ra = q, rb = 63 - q;
        if constexpr (!UPPER) {
            // in fenced groups of 16 loads: formed all at once, the masked
            // offsets of 96 loads would be live beside the values they load
            static_for<0, 32>([&](auto cc) {
                constexpr int c = cc;
                if constexpr (c % 16 == 0) __builtin_amdgcn_sched_barrier(0);
                xa[c] = ident(ra, c, buf_load<T>(rs, off(ra, c)));
            });
            static_for<0, 64>([&](auto cc) {
                constexpr int c = cc;
                if constexpr (c % 16 == 0) __builtin_amdgcn_sched_barrier(0);
                xb[c] = ident(rb, c, buf_load<T>(rs, off(rb, c)));
            });
            __builtin_amdgcn_sched_barrier(0);
        } else {
            // slab sb: rows sb SR .. sb SR + SR - 1 of A, in the columns that
            // reach them (column i >= sb SR); lane q reads row sb SR + q % SR
            // of column u LPI + q / SR.  Entries of a lane's rows right of its
            // diagonal are left as they come (never stored nor used by a
            // referenced entry).
            const int lr = q % SR, lc = q / SR;
            T* tile = lds + CB + h * 64 * PITCH;
            static_for<0, 64 / SR>([&](auto sbc) {
                constexpr int sb = sbc, U0 = sb * SR / LPI, NU = 64 / LPI;
                T st[NU - U0];
                static_for<U0, NU>([&](auto uc) {
                    constexpr int u = uc;
                    st[u - U0] = buf_load<T>(rs, off(u * LPI + opaque_v(lc), sb * SR + opaque_v(lr)));
                });
                T* tw = tile + opaque_v(lc * PITCH + lr);
                static_for<U0, NU>([&](auto uc) {
                    constexpr int u = uc;
                    tw[u * LPI * PITCH] = conj(st[u - U0]);
                });
                wave_lds_sync();
                const T* tra = tile + opaque_v(ra * PITCH);
                const T* trb = tile + opaque_v(rb * PITCH);
                static_for<0, SR>([&](auto rc) {
                    constexpr int c = sb * SR + rc;
                    if constexpr (c < 32) xa[c] = ident(ra, c, tra[rc]);
                    xb[c] = ident(rb, c, trb[rc]);
                });
                wave_lds_sync();
            });
        }

        // Upper: each final column goes into the tile at its step (its
        // registers free at once); after SR steps the tile holds slab sb of
        // the factor, written out as whole lines of A
        auto flush = [&](auto sbc) __attribute__((always_inline)) {
            constexpr int sb = sbc, U0 = sb * SR / LPI, NU = 64 / LPI;
            const int lr = q % SR, lc = q / SR;
            const T* tr = lds + CB + h * 64 * PITCH + opaque_v(lc * PITCH + lr);
            wave_lds_sync();
            static_for<U0, NU>([&](auto uc) {
                constexpr int u = uc;
                buf_store<T>(rs, off(u * LPI + opaque_v(lc), sb * SR + opaque_v(lr)), tr[u * LPI * PITCH]);
            });
            wave_lds_sync();
        };
        int32_t inf = 0;
        colbuf(0, h)[ra] = xa[0];
        colbuf(0, h)[rb] = xb[0];
        wave_lds_sync();
        static_for<0, 64>([&](auto jj) {
            constexpr int j = jj;
            const T* col = colbuf(j & 1, h);
            const R d = re(col[j]);
            inf = (inf == 0 && !(d > R(0))) ? (j + 1) : inf;
            asm volatile("" : "+v"(inf));
            R inv, rsd, sq;
            pivot_terms(d, inv, rsd, sq);
            T ta = zero<T>();
            if constexpr (j < 32) ta = scale(xa[j], inv);
            const T tb = scale(xb[j], inv);
            // column j + 1 first, published for the next step
            if constexpr (j + 1 < 64) {
                const T cj1 = col[j + 1];
                if constexpr (j + 1 < 32) {
                    sub_mul_conj(xa[j + 1], ta, cj1);
                    colbuf((j + 1) & 1, h)[ra] = xa[j + 1];
                }
                sub_mul_conj(xb[j + 1], tb, cj1);
                colbuf((j + 1) & 1, h)[rb] = xb[j + 1];
                wave_lds_sync();
            }
            // the rest: each entry of the column serves both rows of the lane;
            // read in chunks of CH entries, each issued one chunk ahead of the
            // updates that use it, with scheduling fences between chunks (left
            // alone, the compiler reads the whole column ahead and spills)
            constexpr int K0 = j + 2, CH = 32 / int(sizeof(T)) > 0 ? 32 / int(sizeof(T)) : 1;
            if constexpr (K0 < 64) {
                constexpr int NCH = (64 - K0 + CH - 1) / CH;
                T cv[2][CH];
                auto fetch_chunk = [&](auto cc) {
                    constexpr int c = cc;
                    static_for<K0 + c * CH, cmin(64, K0 + (c + 1) * CH)>([&](auto kk) {
                        constexpr int k = kk;
                        cv[c & 1][k - K0 - c * CH] = col[k];
                    });
                };
                fetch_chunk(ic<0>{});
                static_for<0, NCH>([&](auto cc) {
                    constexpr int c = cc;
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (c + 1 < NCH) fetch_chunk(ic<c + 1>{});
                    static_for<K0 + c * CH, cmin(64, K0 + (c + 1) * CH)>([&](auto kk) {
                        constexpr int k = kk;
                        const T ck = cv[c & 1][k - K0 - c * CH];
                        if constexpr (k < 32) sub_mul_conj(xa[k], ta, ck);
                        sub_mul_conj(xb[k], tb, ck);
                    });
                });
                __builtin_amdgcn_sched_barrier(0);
            }
            // column j is final: Lower stores it at once (the column's rows
            // are contiguous), Upper puts it in the tile
            auto fin = [&](int row, const T& v) __attribute__((always_inline)) {
                int r2 = row;
                asm volatile("" : "+v"(r2));
                const T lij = select(r2 == j, diag_value<T>(sq, UPPER), scale(v, rsd));
                if constexpr (UPPER) lds[CB + (h * 64 + r2) * PITCH + j % SR] = conj(lij);
                else buf_store<T>(rs, off(r2, j), lij);
            };
            if constexpr (j < 32) fin(ra, xa[j]);
            fin(rb, xb[j]);
            if constexpr (UPPER && j % SR == SR - 1) flush(ic<j / SR>{});
        });
        if (q == 0 && live && info != nullptr) info[mat] = inf > n ? 0 : inf;
        wave_lds_sync();     // the exchange buffers are reused by the next pair
    }
}

// Every offset inside a pair of matrices (the second one's last element lies
// below two strides) must fit the 31-bit buffer offsets.
template <typename T>
inline bool fold_layout_ok(int64_t stride) { return 2 * stride <= int64_t(0x7fffffff) / int64_t(sizeof(T)); }

template <typename T>
inline void fold_geometry(bool upper, int64_t batch, Geometry& g) {
    g.family = FAM_TINY;
    g.P = 32;
    g.R = 2;
    g.G = 2;
    g.threads = 64;
    g.panel = 0;
    const int64_t pairs = (batch + 1) / 2;
    g.grid = pairs < kFoldMaxGrid ? pairs : kFoldMaxGrid;
    // the pivot buffers; Upper: and the slab tile
    const int64_t es = int64_t(sizeof(T)), pitch = 128 / es + 1;
    g.lds = 2 * 2 * (64 + 4) * es + (upper ? 2 * 64 * pitch * es : 0);
}

template <typename T, bool UPPER>
hipError_t fold_launch(int n, T* a, int64_t lda, int64_t stride, int64_t batch, int32_t* info,
                       hipStream_t s) {
    const int64_t pairs = (batch + 1) / 2;
    const dim3 gd((unsigned)(pairs < kFoldMaxGrid ? pairs : kFoldMaxGrid));
    return launch(potrf_fold_kernel<T, UPPER>, gd, dim3(64), 0, s, a, n, lda, stride, batch, info);
}

}  // namespace fold_detail
}  // namespace bl
