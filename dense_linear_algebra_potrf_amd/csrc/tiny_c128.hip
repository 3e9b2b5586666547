// Tiny-family kernels for element type cdouble (one translation unit per type so
// the kernels build in parallel).  Orders above the register windows run in the
// wide window (tiles over several wavefronts), built in its own translation units.
#include "tiny_impl.hpp"
#include "wide_impl.hpp"

namespace bl {

hipError_t wide_potrf_c128_lower(int n, cdouble* a, int64_t lda, int64_t stride, int64_t batch,
                                 int32_t* info, hipStream_t s);
hipError_t wide_potrf_c128_upper(int n, cdouble* a, int64_t lda, int64_t stride, int64_t batch,
                                 int32_t* info, hipStream_t s);

namespace {
bool wide_order(int n) { return n > tiny_detail::last_nb(tiny_detail::TinyConfigs<cdouble>::type{}); }
}  // namespace

int tiny_max_n_c128() { return wide_detail::kWideMaxOrder; }

bool tiny_layout_ok_c128(int n, int64_t stride) {
    if (wide_order(n)) return wide_detail::wide_layout_ok<cdouble>(stride);
    return tiny_detail::layout_ok_t<cdouble>(n, stride);
}

bool tiny_geometry_c128(bool upper, int n, int64_t lda, int64_t stride, int64_t batch, Geometry& g) {
    if (wide_order(n)) {
        if (n > wide_detail::kWideMaxOrder) return false;
        wide_detail::wide_geometry<cdouble>(upper, n, batch, g);
        return true;
    }
    return tiny_detail::geometry_t<cdouble>(upper, n, lda, stride, batch, g);
}

hipError_t tiny_potrf_c128(bool upper, int n, void* A, int64_t lda, int64_t stride, int64_t batch,
                          int32_t* info, hipStream_t s) {
    if (wide_order(n)) {
        if (n > wide_detail::kWideMaxOrder) return hipErrorInvalidValue;
        cdouble* a = static_cast<cdouble*>(A);
        return upper ? wide_potrf_c128_upper(n, a, lda, stride, batch, info, s)
                     : wide_potrf_c128_lower(n, a, lda, stride, batch, info, s);
    }
    return tiny_detail::potrf_t<cdouble>(upper, n, A, lda, stride, batch, info, s);
}

}  // namespace bl
