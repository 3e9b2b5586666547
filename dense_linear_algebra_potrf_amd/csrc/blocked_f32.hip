// Blocked-family kernels for element type float (one translation unit per type).
#include "blocked_impl.hpp"

namespace bl {

bool blocked_supported_f32(int n, int64_t lda) { return blocked_detail::supported_t<float>(n, lda); }

bool blocked_geometry_f32(int n, int64_t batch, Geometry& g) {
    return blocked_detail::geometry_t<float>(n, batch, g);
}

hipError_t blocked_potrf_f32(bool upper, int n, void* A, int64_t lda, int64_t stride,
                            int64_t batch, int32_t* info, hipStream_t s) {
    return blocked_detail::potrf_t<float>(upper, n, A, lda, stride, batch, info, s);
}

}  // namespace bl
