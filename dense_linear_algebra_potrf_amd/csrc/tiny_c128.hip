// Tiny-family kernels for element type cdouble (one translation unit per type so
// the kernels build in parallel).  Lower 17..32 runs in the folded window (a
// short and a long row per lane), orders above the register windows in the wide
// window (tiles over several wavefronts); both are built in translation units of
// their own.
#include "tiny_impl.hpp"
#include "wide_impl.hpp"
#include "fold_impl.hpp"

namespace bl {

hipError_t wide_potrf_c128_lower(int n, cdouble* a, int64_t lda, int64_t stride, int64_t batch,
                                 int32_t* info, hipStream_t s);
hipError_t wide_potrf_c128_upper(int n, cdouble* a, int64_t lda, int64_t stride, int64_t batch,
                                 int32_t* info, hipStream_t s);
hipError_t fold_potrf_c128(bool upper, int n, cdouble* a, int64_t lda, int64_t stride, int64_t batch,
                           int32_t* info, hipStream_t s);

namespace {
bool wide_order(int n) { return n > tiny_detail::last_nb(tiny_detail::TinyConfigs<cdouble>::type{}); }
// Lower 17..32 in the folded 32-row window where four matrices fit the 31-bit
// offsets: 1.04-1.27x the 32 x 1 window on MI355X at b16384 (Upper there
// 0.96-0.99x, so it keeps 32 x 1)
bool use_fold(bool upper, int n, int64_t stride) {
    return !upper && n >= 17 && n <= 32 && fold_detail::fold_layout_ok<cdouble, 32>(stride);
}
}  // namespace

int tiny_max_n_c128() { return wide_detail::kWideMaxOrder; }

bool tiny_layout_ok_c128(int n, int64_t stride) {
    if (wide_order(n)) return wide_detail::wide_layout_ok<cdouble>(stride);
    return tiny_detail::layout_ok_t<cdouble>(n, stride);
}

bool tiny_geometry_c128(bool upper, int n, int64_t lda, int64_t stride, int64_t batch, Geometry& g) {
    if (use_fold(upper, n, stride)) {
        fold_detail::fold_geometry<cdouble, 32>(upper, batch, g);
        return true;
    }
    if (wide_order(n)) {
        if (n > wide_detail::kWideMaxOrder) return false;
        wide_detail::wide_geometry<cdouble>(upper, n, batch, g);
        return true;
    }
    return tiny_detail::geometry_t<cdouble>(upper, n, lda, stride, batch, g);
}

hipError_t tiny_potrf_c128(bool upper, int n, void* A, int64_t lda, int64_t stride, int64_t batch,
                          int32_t* info, hipStream_t s) {
    if (use_fold(upper, n, stride)) return fold_potrf_c128(upper, n, static_cast<cdouble*>(A), lda, stride, batch, info, s);
    if (wide_order(n)) {
        if (n > wide_detail::kWideMaxOrder) return hipErrorInvalidValue;
        cdouble* a = static_cast<cdouble*>(A);
        return upper ? wide_potrf_c128_upper(n, a, lda, stride, batch, info, s)
                     : wide_potrf_c128_lower(n, a, lda, stride, batch, info, s);
    }
    return tiny_detail::potrf_t<cdouble>(upper, n, A, lda, stride, batch, info, s);
}

}  // namespace bl
