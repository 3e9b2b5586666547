// Tiny-family kernels for element type cdouble (one translation unit per type so
// the kernels build in parallel).
#include "tiny_impl.hpp"

namespace bl {

int tiny_max_n_c128() { return tiny_detail::last_nb(tiny_detail::TinyConfigs<cdouble>::type{}); }

bool tiny_layout_ok_c128(int n, int64_t stride) { return tiny_detail::layout_ok_t<cdouble>(n, stride); }

bool tiny_geometry_c128(bool upper, int n, int64_t lda, int64_t stride, int64_t batch, Geometry& g) {
    return tiny_detail::geometry_t<cdouble>(upper, n, lda, stride, batch, g);
}

hipError_t tiny_potrf_c128(bool upper, int n, void* A, int64_t lda, int64_t stride, int64_t batch,
                          int32_t* info, hipStream_t s) {
    return tiny_detail::potrf_t<cdouble>(upper, n, A, lda, stride, batch, info, s);
}

}  // namespace bl
