// Blocked-family kernels for element type cdouble (one translation unit per type).
#include "blocked_impl.hpp"

namespace bl {

bool blocked_supported_c128(int n, int64_t lda) { return blocked_detail::supported_t<cdouble>(n, lda); }

bool blocked_geometry_c128(int n, int64_t batch, Geometry& g) {
    return blocked_detail::geometry_t<cdouble>(n, batch, g);
}

hipError_t blocked_potrf_c128(bool upper, int n, void* A, int64_t lda, int64_t stride,
                            int64_t batch, int32_t* info, hipStream_t s) {
    return blocked_detail::potrf_t<cdouble>(upper, n, A, lda, stride, batch, info, s);
}

}  // namespace bl
