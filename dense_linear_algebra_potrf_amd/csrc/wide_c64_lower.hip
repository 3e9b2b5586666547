// Wide window of the tiny family: cfloat, Lower (A = L L^H).  One translation unit
// per element type and triangle (each holds large unrolled kernels).
#include "wide_impl.hpp"

namespace bl {

hipError_t wide_potrf_c64_lower(int n, cfloat* a, int64_t lda, int64_t stride, int64_t batch,
                                int32_t* info, hipStream_t s) {
    return wide_detail::wide_launch<cfloat, false>(n, a, lda, stride, batch, info, s);
}

}  // namespace bl
