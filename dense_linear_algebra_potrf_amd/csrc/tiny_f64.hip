// Tiny-family kernels for element type double (one translation unit per type so
// the kernels build in parallel).
#include "tiny_impl.hpp"

namespace bl {

int tiny_max_n_f64() { return tiny_detail::last_nb(tiny_detail::TinyConfigs<double>::type{}); }

bool tiny_layout_ok_f64(int n, int64_t stride) { return tiny_detail::layout_ok_t<double>(n, stride); }

bool tiny_geometry_f64(bool upper, int n, int64_t lda, int64_t stride, int64_t batch, Geometry& g) {
    return tiny_detail::geometry_t<double>(upper, n, lda, stride, batch, g);
}

hipError_t tiny_potrf_f64(bool upper, int n, void* A, int64_t lda, int64_t stride, int64_t batch,
                          int32_t* info, hipStream_t s) {
    return tiny_detail::potrf_t<double>(upper, n, A, lda, stride, batch, info, s);
}

}  // namespace bl
