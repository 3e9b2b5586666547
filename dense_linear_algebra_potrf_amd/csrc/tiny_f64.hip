// Tiny-family kernels for element type double (one translation unit per type so
// the kernels build in parallel).  Orders 25..64 run in the folded window (a
// short and a long row per lane), orders above the register windows in the
// wide window (tiles over several wavefronts); both are built in translation
// units of their own.
#include "tiny_impl.hpp"
#include "wide_impl.hpp"
#include "fold_impl.hpp"

namespace bl {

hipError_t wide_potrf_f64_lower(int n, double* a, int64_t lda, int64_t stride, int64_t batch,
                                int32_t* info, hipStream_t s);
hipError_t wide_potrf_f64_upper(int n, double* a, int64_t lda, int64_t stride, int64_t batch,
                                int32_t* info, hipStream_t s);
hipError_t fold_potrf_f64(bool upper, int n, double* a, int64_t lda, int64_t stride, int64_t batch,
                          int32_t* info, hipStream_t s);

namespace {
bool wide_order(int n) { return n > tiny_detail::last_nb(tiny_detail::TinyConfigs<double>::type{}); }
// orders 25..64 in the folded window where its wavefront's matrices fit the
// 31-bit offsets (else the register windows): 25..32 in the 32-row window
// (1.13-1.29x the 8 x 4 window on MI355X at b16384), 33..48 in the 48-row
// window (1.23-1.39x the 64-row one), the rest in the 64-row one (a 56-row
// window, without DPP updates since 56 rows are not whole groups of 16,
// measured 0.91-0.95x at 49..56)
bool use_fold(int n, int64_t stride) {
    if (n >= 25 && n <= 32) return fold_detail::fold_layout_ok<double, 32>(stride);
    return n >= fold_detail::kFoldMin && n <= fold_detail::kFoldMax && fold_detail::fold_layout_ok<double, 64>(stride);
}
}  // namespace

int tiny_max_n_f64() { return wide_detail::kWideMaxOrder; }

bool tiny_layout_ok_f64(int n, int64_t stride) {
    if (wide_order(n)) return wide_detail::wide_layout_ok<double>(stride);
    if (use_fold(n, stride)) return true;
    return tiny_detail::layout_ok_t<double>(n, stride);
}

bool tiny_geometry_f64(bool upper, int n, int64_t lda, int64_t stride, int64_t batch, Geometry& g) {
    if (wide_order(n)) {
        if (n > wide_detail::kWideMaxOrder) return false;
        wide_detail::wide_geometry<double>(upper, n, batch, g);
        return true;
    }
    if (use_fold(n, stride)) {
        if (n <= 32) fold_detail::fold_geometry<double, 32>(upper, batch, g);
        else if (n <= 48) fold_detail::fold_geometry<double, 48>(upper, batch, g);
        else fold_detail::fold_geometry<double, 64>(upper, batch, g);
        return true;
    }
    return tiny_detail::geometry_t<double>(upper, n, lda, stride, batch, g);
}

hipError_t tiny_potrf_f64(bool upper, int n, void* A, int64_t lda, int64_t stride, int64_t batch,
                          int32_t* info, hipStream_t s) {
    if (wide_order(n)) {
        if (n > wide_detail::kWideMaxOrder) return hipErrorInvalidValue;
        double* a = static_cast<double*>(A);
        return upper ? wide_potrf_f64_upper(n, a, lda, stride, batch, info, s)
                     : wide_potrf_f64_lower(n, a, lda, stride, batch, info, s);
    }
    if (use_fold(n, stride)) return fold_potrf_f64(upper, n, static_cast<double*>(A), lda, stride, batch, info, s);
    return tiny_detail::potrf_t<double>(upper, n, A, lda, stride, batch, info, s);
}

}  // namespace bl
