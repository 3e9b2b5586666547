// Tiny-family kernels for element type cfloat (one translation unit per type so
// the kernels build in parallel).  Orders 33..64 run in the folded window (two
// matrices per wavefront, a short and a long row per lane), orders above the
// register windows in the wide window (tiles over several wavefronts); both are
// built in translation units of their own.
#include "tiny_impl.hpp"
#include "wide_impl.hpp"
#include "fold_impl.hpp"

namespace bl {

hipError_t wide_potrf_c64_lower(int n, cfloat* a, int64_t lda, int64_t stride, int64_t batch,
                                int32_t* info, hipStream_t s);
hipError_t wide_potrf_c64_upper(int n, cfloat* a, int64_t lda, int64_t stride, int64_t batch,
                                int32_t* info, hipStream_t s);
hipError_t fold_potrf_c64(bool upper, int n, cfloat* a, int64_t lda, int64_t stride, int64_t batch,
                          int32_t* info, hipStream_t s);

namespace {
bool wide_order(int n) { return n > tiny_detail::last_nb(tiny_detail::TinyConfigs<cfloat>::type{}); }
// orders 33..64 in the folded window where a pair of matrices fits its 31-bit
// offsets (else the one-wavefront window): up to 48 in the 48-row window
// (1.40-1.51x the 64-row one on MI355X at b16384), 49..56 in the 56-row window
// (1.15-1.19x), the rest in the 64-row one
bool use_fold(int n, int64_t stride) {
    return n >= fold_detail::kFoldMin && n <= fold_detail::kFoldMax && fold_detail::fold_layout_ok<cfloat, 64>(stride);
}
}  // namespace

int tiny_max_n_c64() { return wide_detail::kWideMaxOrder; }

bool tiny_layout_ok_c64(int n, int64_t stride) {
    if (wide_order(n)) return wide_detail::wide_layout_ok<cfloat>(stride);
    if (use_fold(n, stride)) return true;
    return tiny_detail::layout_ok_t<cfloat>(n, stride);
}

bool tiny_geometry_c64(bool upper, int n, int64_t lda, int64_t stride, int64_t batch, Geometry& g) {
    if (wide_order(n)) {
        if (n > wide_detail::kWideMaxOrder) return false;
        wide_detail::wide_geometry<cfloat>(upper, n, batch, g);
        return true;
    }
    if (use_fold(n, stride)) {
        if (n <= 48) fold_detail::fold_geometry<cfloat, 48>(upper, batch, g);
        else if (n <= 56) fold_detail::fold_geometry<cfloat, 56>(upper, batch, g);
        else fold_detail::fold_geometry<cfloat, 64>(upper, batch, g);
        return true;
    }
    return tiny_detail::geometry_t<cfloat>(upper, n, lda, stride, batch, g);
}

hipError_t tiny_potrf_c64(bool upper, int n, void* A, int64_t lda, int64_t stride, int64_t batch,
                          int32_t* info, hipStream_t s) {
    if (wide_order(n)) {
        if (n > wide_detail::kWideMaxOrder) return hipErrorInvalidValue;
        cfloat* a = static_cast<cfloat*>(A);
        return upper ? wide_potrf_c64_upper(n, a, lda, stride, batch, info, s)
                     : wide_potrf_c64_lower(n, a, lda, stride, batch, info, s);
    }
    if (use_fold(n, stride)) return fold_potrf_c64(upper, n, static_cast<cfloat*>(A), lda, stride, batch, info, s);
    return tiny_detail::potrf_t<cfloat>(upper, n, A, lda, stride, batch, info, s);
}

}  // namespace bl
