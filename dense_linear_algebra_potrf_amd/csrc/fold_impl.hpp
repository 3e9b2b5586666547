// Folded window of the tiny family (implementation header): a window of NB rows
// held by NB / 2 lanes per matrix, lane q holding rows q and NB - 1 - q:
// NB = 34 (17 lanes per matrix, three matrices per wavefront), NB = 48 (24
// lanes of a 32-lane group, two), NB = 64 (two) and NB = 128 (one).
//
// Prior art: the BatchLAS perf_potrf page, section "potrf: the tiny tier" (lane
// r owns row r, every value in registers) and section "The LPanel tier" (one
// thread per row at mid orders).  With one row per lane every lane updates
// every column right of the pivot, while row i only has columns up to i: half
// of the updates land in entries that are never stored.  Folding the rows
// pairs a short row with a long one: row q keeps columns 0 .. NB/2 - 1 and row
// NB - 1 - q columns 0 .. NB - 1, so at step j a lane updates
// (NB/2 - 1 - j) + (NB - 1 - j) entries for two rows where a row per lane
// updates NB - 1 - j for one, about a third fewer updates per matrix.  At
// NB = 128 it also keeps a matrix inside one wavefront (no workgroup barrier
// per column).  The recurrence is the tiny family's (right-looking, the Schur
// pivot never stale, the multiplier s_ij / d on the unscaled column, failures
// as selects); the pivot column goes through LDS, double-buffered by step
// parity, one buffer per matrix, with no barrier inside the wavefront.  For the
// real types with rows of 16 lanes inside a matrix the updates take the
// column's entries by DPP row broadcasts: lane q reads entry 16 g + (q mod 16)
// of group g, and each multiply-add takes entry k from lane k mod 16 of its row
// of 16 lanes, so one LDS read serves 16 entries for both of the lane's rows.
// Rows at or beyond n hold the identity, so the steps past n see d = 1.  The
// routes (which window serves which type, triangle and order) are chosen by
// the tiny family's per-type translation units from measurements.
#pragma once

#include "families.hpp"
#include "wide_impl.hpp"

namespace bl {
namespace fold_detail {

constexpr int kFoldMin = 33, kFoldMax = 64;               // the fp64 and cfloat orders (fp32 routes its own)
constexpr int64_t kFoldMaxGrid = int64_t(1) << 19;     // workgroups of one wavefront

template <int NB> constexpr int fold_half() { return NB / 2; }          // lanes holding rows of a matrix
// lanes per matrix group: NB / 2, except that the 48- and 56-row windows take
// groups of 32 lanes (8 and 4 idle), so that a DPP row of 16 lanes never spans
// two matrices
template <int NB> constexpr int fold_gsize() { return NB == 48 || NB == 56 ? 32 : NB / 2; }
template <int NB> constexpr int fold_mpw() { return 64 / fold_gsize<NB>(); }    // matrices per wavefront
// lane groups in a wavefront, an idle tail included (each has its pivot
// buffers, so idle lanes need no guard)
template <int NB> constexpr int fold_groups() { return (64 + fold_gsize<NB>() - 1) / fold_gsize<NB>(); }
// slots of a pivot buffer: the NB rows, two spare slots per idle lane of a
// group, padding
template <int NB> constexpr int fold_slot() { return NB + 2 * (fold_gsize<NB>() - NB / 2) + 4; }
// rows of A in a slab: one 128-byte line of a column, or half a line where
// whole lines do not divide the window or its lane group (fp32 at 32 and 48
// rows, 8-byte types at 56)
template <typename T, int NB>
constexpr int fold_slab_rows() {
    return NB % (128 / int(sizeof(T))) == 0 && fold_gsize<NB>() % (128 / int(sizeof(T))) == 0
               ? 128 / int(sizeof(T)) : 64 / int(sizeof(T));
}
// occupancy asked of the compiler, from the registers a lane's values take:
// up to 51 (the fp32 34-row window) six wavefronts per SIMD, up to 72 four,
// more two (144 registers of values at three wavefronts spilled)
template <typename T, int NB>
constexpr int fold_value_regs() { return (3 * NB / 2) * int(sizeof(T)) / 4; }
template <typename T, int NB>
constexpr int fold_waves_per_eu() {
    return fold_value_regs<T, NB>() <= 51 ? 6 : fold_value_regs<T, NB>() <= 72 ? 4 : 2;
}
// rows of a matrix's slab tile (Upper): the NB rows and two spare rows per
// idle lane of a group
template <int NB> constexpr int fold_tile_rows() { return NB + 2 * (fold_gsize<NB>() - NB / 2); }
// LDS elements: the pivot buffers, and for Upper the slab tile
template <typename T, int NB, bool UPPER>
constexpr int fold_lds_elems() {
    return 2 * fold_groups<NB>() * fold_slot<NB>() +
           (UPPER ? fold_mpw<NB>() * fold_tile_rows<NB>() * (fold_slab_rows<T, NB>() + 1) : 0);
}

// An opaque copy: the column and row indices of the slab passes are shared by
// the loads and the stores; formed once, all of them would be held across the
// factorisation.
__device__ __forceinline__ int opaque_v(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

template <typename T, int NB, bool UPPER>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(fold_waves_per_eu<T, NB>()))) void potrf_fold_kernel(
    T* __restrict__ A, int n, int64_t lda, int64_t stride, int64_t batch, int32_t* __restrict__ info)
{
    using R = typename Traits<T>::R;
    constexpr uint32_t S = sizeof(T);
    constexpr int HALF = fold_half<NB>(), GS = fold_gsize<NB>(), MPW = fold_mpw<NB>();
    // Upper: lane q's rows are columns of A, so loads and stores per row would
    // touch a cache line per lane and element.  The referenced triangle
    // instead moves in slabs of SR rows of A (SR elements = one 128-byte line
    // of a column, or half of one): each instruction covers whole lines (LPI
    // columns per matrix), the slab is transposed through a tile of NB columns
    // per matrix (a column's SR elements plus one element of padding; spare
    // rows for idle lanes), and every lane picks its two columns out of it.
    // A slab of the factor is written as soon as its SR columns are final.
    constexpr int SR = fold_slab_rows<T, NB>(), LPI = GS / SR > 0 ? GS / SR : 1, PITCH = SR + 1;
    constexpr int TR = fold_tile_rows<NB>();
    constexpr int GROUPS = fold_groups<NB>(), SLOT = fold_slot<NB>(), CB = 2 * GROUPS * SLOT;
    // DPP broadcasts need rows of 16 lanes within one matrix
    constexpr bool DPP = !Traits<T>::cplx && GS % 16 == 0 && NB % 16 == 0;
    static_assert(NB % 2 == 0 && HALF <= GS && GS <= 64, "fold geometry");
    static_assert(!UPPER || (64 % GS == 0 && GS % SR == 0 && NB % SR == 0), "Upper slab geometry");
    static_assert((HALF + NB) * int(S) <= 192 * 4, "two rows per lane in 192 registers");
    __shared__ __attribute__((aligned(16))) T lds[fold_lds_elems<T, NB, UPPER>()];
    auto colbuf = [&](int par, int mh) __attribute__((always_inline)) { return lds + (par * GROUPS + mh) * SLOT; };

    const int lane = threadIdx.x & 63;
    const int h = lane / GS;                  // which matrix of the wavefront
    const int q = lane % GS;
    const bool own = q < HALF;                // (the 48- and 56-row windows' groups end in idle lanes)
    const int q16 = lane & 15;                // lane within its row of 16 (DPP broadcasts)
    const uint32_t lda_b = uint32_t(lda) * S;

    for (int64_t m0 = MPW * int64_t(blockIdx.x); m0 < batch; m0 += MPW * int64_t(gridDim.x)) {
        const int64_t mat = m0 + h;
        const bool live = h < MPW && mat < batch;    // (lanes past MPW groups are idle)
        // one descriptor for the wavefront's matrices (a descriptor must be the
        // same for the whole wavefront), matrix h at a byte offset inside it
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(A + m0 * stride);
        const uint32_t mbase = uint32_t(h) * uint32_t(stride) * S;
        // row `row`'s element of column c (out of range: masked), behind an
        // opaque copy of the row so that nothing derived from it is held
        // across the factorisation
        auto off = [&](int row, int c) __attribute__((always_inline)) {
            asm volatile("" : "+v"(row));
            uint32_t ldb = lda_b;            // (the column offsets are formed where used)
            asm volatile("" : "+s"(ldb));
            int lim = live && (UPPER || own) ? n : 0;   // a missing matrix (or an idle lane) has no rows
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
        T xa[HALF], xb[NB];
        const int ra = q, rb = NB - 1 - q;
        // pivot-buffer slots written: the two rows, or an idle lane's spares
        const int wa = own ? ra : NB + 2 * (q - HALF), wb = own ? rb : NB + 2 * (q - HALF) + 1;
        if constexpr (!UPPER) {
            // in fenced groups of 16 loads (8 for 16-byte elements): formed
            // all at once, the masked offsets of every load would be live
            // beside the values they load
            constexpr int LG = S >= 16 ? 8 : 16;
            static_for<0, HALF>([&](auto cc) {
                constexpr int c = cc;
                if constexpr (c % LG == 0) __builtin_amdgcn_sched_barrier(0);
                xa[c] = ident(ra, c, buf_load<T>(rs, off(ra, c)));
            });
            static_for<0, NB>([&](auto cc) {
                constexpr int c = cc;
                if constexpr (c % LG == 0) __builtin_amdgcn_sched_barrier(0);
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
            T* tile = lds + CB + h * TR * PITCH;
            static_for<0, NB / SR>([&](auto sbc) {
                constexpr int sb = sbc, U0 = sb * SR / LPI, NU = NB / LPI;
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
                    if constexpr (c < HALF) xa[c] = ident(ra, c, tra[rc]);
                    xb[c] = ident(rb, c, trb[rc]);
                });
                wave_lds_sync();
            });
        }

        // Upper: each final column goes into the tile at its step (its
        // registers free at once); after SR steps the tile holds slab sb of
        // the factor, written out as whole lines of A
        auto flush = [&](auto sbc) __attribute__((always_inline)) {
            constexpr int sb = sbc, U0 = sb * SR / LPI, NU = NB / LPI;
            const int lr = q % SR, lc = q / SR;
            const T* tr = lds + CB + h * TR * PITCH + opaque_v(lc * PITCH + lr);
            wave_lds_sync();
            static_for<U0, NU>([&](auto uc) {
                constexpr int u = uc;
                buf_store<T>(rs, off(u * LPI + opaque_v(lc), sb * SR + opaque_v(lr)), tr[u * LPI * PITCH]);
            });
            wave_lds_sync();
        };
        int32_t inf = 0;
        colbuf(0, h)[wa] = xa[0];
        colbuf(0, h)[wb] = xb[0];
        wave_lds_sync();
        static_for<0, NB>([&](auto jj) {
            constexpr int j = jj;
            const T* col = colbuf(j & 1, h);
            const R d = re(col[j]);
            wide_detail::note_pivot(inf, d, j);
            R inv, rsd, sq;
            pivot_terms(d, inv, rsd, sq);
            T ta = zero<T>();
            if constexpr (j < HALF) ta = scale(xa[j], inv);
            const T tb = scale(xb[j], inv);
            // column j + 1 first, published for the next step
            if constexpr (j + 1 < NB) {
                const T cj1 = col[j + 1];
                if constexpr (j + 1 < HALF) {
                    sub_mul_conj(xa[j + 1], ta, cj1);
                    colbuf((j + 1) & 1, h)[wa] = xa[j + 1];
                }
                sub_mul_conj(xb[j + 1], tb, cj1);
                colbuf((j + 1) & 1, h)[wb] = xb[j + 1];
                wave_lds_sync();
            }
            // the rest.  Real types with rows of 16 lanes in one matrix: group
            // by group of 16 entries by DPP row broadcasts, each group's read
            // issued one group ahead of its updates.  Otherwise every lane
            // reads the entries, in chunks of 32 bytes, each chunk one ahead
            // of its updates, with scheduling fences between chunks (left
            // alone, the compiler reads the whole column ahead and spills);
            // the four multiply-adds of a complex update measured slower as
            // DPP broadcasts.
            constexpr int K0 = j + 2;
            if constexpr (!DPP && K0 < NB) {
                // chunks of 32 bytes; 16 at six wavefronts per SIMD and for
                // cdouble (one element), which keep those windows spill-free
                constexpr int CH = (fold_waves_per_eu<T, NB>() >= 6 || S >= 16) ? 16 / int(S) : 32 / int(S);
                constexpr int NCH = (NB - K0 + CH - 1) / CH;
                T cv[2][CH];
                auto fetch_chunk = [&](auto cc) __attribute__((always_inline)) {
                    constexpr int c = cc;
                    static_for<K0 + c * CH, cmin(NB, K0 + (c + 1) * CH)>([&](auto kk) {
                        constexpr int k = kk;
                        cv[c & 1][k - K0 - c * CH] = col[k];
                    });
                };
                fetch_chunk(ic<0>{});
                static_for<0, NCH>([&](auto cc) {
                    constexpr int c = cc;
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (c + 1 < NCH) fetch_chunk(ic<c + 1>{});
                    static_for<K0 + c * CH, cmin(NB, K0 + (c + 1) * CH)>([&](auto kk) {
                        constexpr int k = kk;
                        const T ck = cv[c & 1][k - K0 - c * CH];
                        if constexpr (k < HALF) sub_mul_conj(xa[k], ta, ck);
                        sub_mul_conj(xb[k], tb, ck);
                    });
                });
                __builtin_amdgcn_sched_barrier(0);
            } else if constexpr (K0 < NB) {
                constexpr int G0 = K0 / 16, G1 = NB / 16;
                const auto ma = wide_detail::wide_mult(ta);
                const auto mb = wide_detail::wide_mult(tb);
                const T* colq = col + q16;
                T cg[2];
                cg[G0 & 1] = colq[16 * G0];
                static_for<G0, G1>([&](auto gg) {
                    constexpr int g = gg;
                    if constexpr (g + 1 < G1) cg[(g + 1) & 1] = colq[16 * (g + 1)];
                    constexpr int KB = cmax(K0, 16 * g);
                    static_for<KB, 16 * g + 16>([&](auto kk) {
                        constexpr int k = kk;
                        wide_detail::wide_fma16<k - 16 * g, k == KB>(xb[k], mb, cg[g & 1]);
                        if constexpr (k < HALF)
                            wide_detail::wide_fma16<k - 16 * g, false>(xa[k], ma, cg[g & 1]);
                    });
                });
            }
            // column j is final: Lower stores it at once (the column's rows
            // are contiguous), Upper puts it in the tile (row slot: the row,
            // or an idle lane's spare)
            auto fin = [&](int row, int slot, const T& v) __attribute__((always_inline)) {
                int r2 = row;
                asm volatile("" : "+v"(r2));
                const T lij = select(r2 == j, diag_value<T>(sq, UPPER), scale(v, rsd));
                if constexpr (UPPER) lds[CB + (h * TR + slot) * PITCH + j % SR] = conj(lij);
                else buf_store<T>(rs, off(r2, j), lij);
            };
            if constexpr (j < HALF) fin(ra, wa, xa[j]);
            fin(rb, wb, xb[j]);
            if constexpr (UPPER && j % SR == SR - 1) flush(ic<j / SR>{});
        });
        if (q == 0 && live && info != nullptr) info[mat] = inf > n ? 0 : inf;
        wave_lds_sync();     // the exchange buffers are reused by the next matrices
    }
}

// Every offset inside a wavefront's matrices (the last one's last element lies
// below MPW strides) must fit the 31-bit buffer offsets.
template <typename T, int NB>
inline bool fold_layout_ok(int64_t stride) {
    return int64_t(fold_mpw<NB>()) * stride <= int64_t(0x7fffffff) / int64_t(sizeof(T));
}

template <typename T, int NB>
inline void fold_geometry(bool upper, int64_t batch, Geometry& g) {
    constexpr int MPW = fold_mpw<NB>();
    g.family = FAM_TINY;
    g.P = fold_half<NB>();
    g.R = 2;
    g.G = MPW;
    g.threads = 64;
    g.panel = 0;
    const int64_t waves = (batch + MPW - 1) / MPW;
    g.grid = waves < kFoldMaxGrid ? waves : kFoldMaxGrid;
    g.lds = int64_t(upper ? fold_lds_elems<T, NB, true>() : fold_lds_elems<T, NB, false>()) *
            int64_t(sizeof(T));
}

template <typename T, int NB, bool UPPER>
hipError_t fold_launch(int n, T* a, int64_t lda, int64_t stride, int64_t batch, int32_t* info,
                       hipStream_t s) {
    constexpr int MPW = fold_mpw<NB>();
    const int64_t waves = (batch + MPW - 1) / MPW;
    const dim3 gd((unsigned)(waves < kFoldMaxGrid ? waves : kFoldMaxGrid));
    return launch(potrf_fold_kernel<T, NB, UPPER>, gd, dim3(64), 0, s, a, n, lda, stride, batch, info);
}

}  // namespace fold_detail
}  // namespace bl
