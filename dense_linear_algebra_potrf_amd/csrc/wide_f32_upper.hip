// Wide fp32 window of the tiny family, Upper (A = U^H U) (one translation unit
// per triangle: each holds large unrolled kernels).
#include "wide_impl.hpp"

namespace bl {

hipError_t wide_potrf_f32_upper(int n, float* a, int64_t lda, int64_t stride, int64_t batch,
                             int32_t* info, hipStream_t s) {
    return wide_detail::wide_launch<true>(n, a, lda, stride, batch, info, s);
}

}  // namespace bl
