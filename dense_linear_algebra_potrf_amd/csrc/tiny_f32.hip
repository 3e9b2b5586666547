// Tiny-family kernels for element type float (one translation unit per type so
// the kernels build in parallel).  Orders above the register windows run in the
// wide window (two wavefronts per matrix), built in its own translation units.
#include "tiny_impl.hpp"
#include "wide_impl.hpp"

namespace bl {

hipError_t wide_potrf_f32_lower(int n, float* a, int64_t lda, int64_t stride, int64_t batch,
                                int32_t* info, hipStream_t s);
hipError_t wide_potrf_f32_upper(int n, float* a, int64_t lda, int64_t stride, int64_t batch,
                                int32_t* info, hipStream_t s);

namespace {
bool wide_order(int n) { return n > tiny_detail::last_nb(tiny_detail::TinyConfigs<float>::type{}); }
}  // namespace

int tiny_max_n_f32() { return wide_detail::kWideMaxOrder; }

bool tiny_layout_ok_f32(int n, int64_t stride) {
    if (wide_order(n)) return wide_detail::wide_layout_ok<float>(stride);
    return tiny_detail::layout_ok_t<float>(n, stride);
}

bool tiny_geometry_f32(bool upper, int n, int64_t lda, int64_t stride, int64_t batch, Geometry& g) {
    if (wide_order(n)) {
        if (n > wide_detail::kWideMaxOrder) return false;
        wide_detail::wide_geometry<float>(n, batch, g);
        return true;
    }
    return tiny_detail::geometry_t<float>(upper, n, lda, stride, batch, g);
}

hipError_t tiny_potrf_f32(bool upper, int n, void* A, int64_t lda, int64_t stride, int64_t batch,
                          int32_t* info, hipStream_t s) {
    if (wide_order(n)) {
        if (n > wide_detail::kWideMaxOrder) return hipErrorInvalidValue;
        float* a = static_cast<float*>(A);
        return upper ? wide_potrf_f32_upper(n, a, lda, stride, batch, info, s)
                     : wide_potrf_f32_lower(n, a, lda, stride, batch, info, s);
    }
    return tiny_detail::potrf_t<float>(upper, n, A, lda, stride, batch, info, s);
}

}  // namespace bl
