// Blocked-family kernels for element type cfloat (one translation unit per type).
#include "blocked_impl.hpp"

namespace bl {

bool blocked_supported_c64(int n, int64_t lda) { return blocked_detail::supported_t<cfloat>(n, lda); }

bool blocked_geometry_c64(int n, int64_t batch, Geometry& g) {
    return blocked_detail::geometry_t<cfloat>(n, batch, g);
}

hipError_t blocked_potrf_c64(bool upper, int n, void* A, int64_t lda, int64_t stride,
                            int64_t batch, int32_t* info, hipStream_t s) {
    return blocked_detail::potrf_t<cfloat>(upper, n, A, lda, stride, batch, info, s);
}

}  // namespace bl
