// Fused posv kernels (tiny family) for element type cfloat.
#include "tiny_impl.hpp"

namespace bl {

int posv_tiny_max_n_c64() { return tiny_detail::last_nb(tiny_detail::PosvConfigs<cfloat>::type{}); }

bool posv_tiny_geometry_c64(bool upper, int n, int64_t lda, int64_t stride, int64_t batch, Geometry& g) {
    return tiny_detail::geometry_t<cfloat, tiny_detail::PosvConfigs<cfloat>::type>(upper, n, lda, stride, batch, g);
}

bool posv_tiny_layout_ok_c64(int n, int64_t strideA, int64_t strideB) {
    return tiny_detail::posv_layout_ok_t<cfloat>(n, strideA, strideB);
}

hipError_t posv_tiny_c64(bool upper, int n, int nrhs, void* A, int64_t lda, int64_t strideA,
                         void* B, int64_t ldb, int64_t strideB, int64_t batch, int32_t* info,
                         hipStream_t s) {
    return tiny_detail::posv_t<cfloat>(upper, n, nrhs, A, lda, strideA, B, ldb, strideB, batch, info, s);
}

}  // namespace bl
