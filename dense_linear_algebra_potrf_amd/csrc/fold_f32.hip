// Folded window of the tiny family: float, where it measured faster than the
// window it replaces (Upper at 25..32, four matrices per wavefront; Lower at
// order 34, three; 35..48 both triangles and Lower 49..64, two; Upper at
// 97..128, one).
#include "fold_impl.hpp"

namespace bl {

hipError_t fold_potrf_f32(bool upper, int n, float* a, int64_t lda, int64_t stride, int64_t batch,
                          int32_t* info, hipStream_t s) {
    if (upper && n <= 32) return fold_detail::fold_launch<float, 32, true>(n, a, lda, stride, batch, info, s);
    if (!upper && n <= 34) return fold_detail::fold_launch<float, 34, false>(n, a, lda, stride, batch, info, s);
    if (n <= 48)
        return upper ? fold_detail::fold_launch<float, 48, true>(n, a, lda, stride, batch, info, s)
                     : fold_detail::fold_launch<float, 48, false>(n, a, lda, stride, batch, info, s);
    if (!upper && n <= 64) return fold_detail::fold_launch<float, 64, false>(n, a, lda, stride, batch, info, s);
    if (upper && n > 64) return fold_detail::fold_launch<float, 128, true>(n, a, lda, stride, batch, info, s);
    return hipErrorInvalidValue;
}

}  // namespace bl
