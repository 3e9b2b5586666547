// Tiny-family kernels for element type float (one translation unit per type so
// the kernels build in parallel).  Orders above the register windows run in the
// wide window (two wavefronts per matrix), built in its own translation units.
#include "tiny_impl.hpp"
#include "wide_impl.hpp"
#include "fold_impl.hpp"

namespace bl {

hipError_t wide_potrf_f32_lower(int n, float* a, int64_t lda, int64_t stride, int64_t batch,
                                int32_t* info, hipStream_t s);
hipError_t wide_potrf_f32_upper(int n, float* a, int64_t lda, int64_t stride, int64_t batch,
                                int32_t* info, hipStream_t s);
hipError_t fold_potrf_f32(bool upper, int n, float* a, int64_t lda, int64_t stride, int64_t batch,
                          int32_t* info, hipStream_t s);

namespace {
bool wide_order(int n) { return n > tiny_detail::last_nb(tiny_detail::TinyConfigs<float>::type{}); }
// The folded window where it measured faster on MI355X (b16384, against the
// window it replaces): Upper 25..32 in the 32-row window (1.03-1.35x the
// 16 x 2 window; Lower there 0.83-0.88x), Lower 34 in the 34-row window (1.6x the 64-row one;
// order 33 keeps its 11 x 3 window, 44.5 against 51.7 us), 35..48 in the
// 48-row window (Lower 1.29-1.43x the 64-row one, Upper 1.52-1.76x the 64 x 1
// window), Lower 49..64 in the 64-row window (1.06-1.23x the 64 x 1 window;
// Upper there 0.93-0.95x), Upper
// 97..128 in the 128-row window (1.27-1.62x the rows layout with per-row Upper
// accesses, 1.03-1.08x with its slab tile; Lower there 0.55-0.60x, the rows
// layout already skipping the triangle per wavefront), and only where a
// wavefront's matrices fit the 31-bit offsets.
bool use_fold(bool upper, int n, int64_t stride) {
    if (upper && n >= 25 && n <= 32) return fold_detail::fold_layout_ok<float, 32>(stride);
    if (!upper && n == 34) return fold_detail::fold_layout_ok<float, 34>(stride);
    if (n >= 35 && n <= 48) return fold_detail::fold_layout_ok<float, 48>(stride);
    if (!upper && n >= 49 && n <= 64) return fold_detail::fold_layout_ok<float, 64>(stride);
    if (upper && n >= 97 && n <= 128) return fold_detail::fold_layout_ok<float, 128>(stride);
    return false;
}
}  // namespace

int tiny_max_n_f32() { return wide_detail::kWideMaxOrder; }

bool tiny_layout_ok_f32(int n, int64_t stride) {
    if (wide_order(n)) return wide_detail::wide_layout_ok<float>(stride);
    return tiny_detail::layout_ok_t<float>(n, stride);
}

bool tiny_geometry_f32(bool upper, int n, int64_t lda, int64_t stride, int64_t batch, Geometry& g) {
    if (use_fold(upper, n, stride)) {
        if (n <= 32) fold_detail::fold_geometry<float, 32>(upper, batch, g);
        else if (n <= 34) fold_detail::fold_geometry<float, 34>(upper, batch, g);
        else if (n <= 48) fold_detail::fold_geometry<float, 48>(upper, batch, g);
        else if (n <= 64) fold_detail::fold_geometry<float, 64>(upper, batch, g);
        else fold_detail::fold_geometry<float, 128>(upper, batch, g);
        return true;
    }
    if (wide_order(n)) {
        if (n > wide_detail::kWideMaxOrder) return false;
        wide_detail::wide_geometry<float>(upper, n, batch, g);
        return true;
    }
    return tiny_detail::geometry_t<float>(upper, n, lda, stride, batch, g);
}

hipError_t tiny_potrf_f32(bool upper, int n, void* A, int64_t lda, int64_t stride, int64_t batch,
                          int32_t* info, hipStream_t s) {
    if (use_fold(upper, n, stride)) return fold_potrf_f32(upper, n, static_cast<float*>(A), lda, stride, batch, info, s);
    if (wide_order(n)) {
        if (n > wide_detail::kWideMaxOrder) return hipErrorInvalidValue;
        float* a = static_cast<float*>(A);
        return upper ? wide_potrf_f32_upper(n, a, lda, stride, batch, info, s)
                     : wide_potrf_f32_lower(n, a, lda, stride, batch, info, s);
    }
    return tiny_detail::potrf_t<float>(upper, n, A, lda, stride, batch, info, s);
}

}  // namespace bl
