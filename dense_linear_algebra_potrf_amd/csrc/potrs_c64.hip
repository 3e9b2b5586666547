// Triangular solves of the split posv route for element type cfloat (one
// translation unit per type).
#include "potrs_impl.hpp"

namespace bl {

bool potrs_supported_c64(int n, int nrhs) { return potrs_detail::supported_t<cfloat>(n, nrhs); }

hipError_t potrs_c64(bool upper, int n, int nrhs, const void* A, int64_t lda, int64_t strideA,
                     void* B, int64_t ldb, int64_t strideB, int64_t batch, const int32_t* info,
                     hipStream_t s) {
    return potrs_detail::potrs_t<cfloat>(upper, n, nrhs, A, lda, strideA, B, ldb, strideB, batch, info, s);
}

}  // namespace bl
