// Blocked-family kernels for element type double (one translation unit per type).
#include "blocked_impl.hpp"

namespace bl {

bool blocked_supported_f64(int n, int64_t lda) { return blocked_detail::supported_t<double>(n, lda); }

bool blocked_geometry_f64(int n, int64_t batch, Geometry& g) {
    return blocked_detail::geometry_t<double>(n, batch, g);
}

hipError_t blocked_potrf_f64(bool upper, int n, void* A, int64_t lda, int64_t stride,
                            int64_t batch, int32_t* info, hipStream_t s) {
    return blocked_detail::potrf_t<double>(upper, n, A, lda, stride, batch, info, s);
}

}  // namespace bl
