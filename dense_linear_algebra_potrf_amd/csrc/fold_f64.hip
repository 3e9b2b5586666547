// Folded window of the tiny family: double, both triangles, a short and a long
// row per lane (orders 25..32 in the 32-row window, four matrices per
// wavefront; 33..48 in the 48-row window and 49..64 in the 64-row one, two).
#include "fold_impl.hpp"

namespace bl {

hipError_t fold_potrf_f64(bool upper, int n, double* a, int64_t lda, int64_t stride, int64_t batch,
                          int32_t* info, hipStream_t s) {
    if (n <= 32)
        return upper ? fold_detail::fold_launch<double, 32, true>(n, a, lda, stride, batch, info, s)
                     : fold_detail::fold_launch<double, 32, false>(n, a, lda, stride, batch, info, s);
    if (n <= 48)
        return upper ? fold_detail::fold_launch<double, 48, true>(n, a, lda, stride, batch, info, s)
                     : fold_detail::fold_launch<double, 48, false>(n, a, lda, stride, batch, info, s);
    return upper ? fold_detail::fold_launch<double, 64, true>(n, a, lda, stride, batch, info, s)
                 : fold_detail::fold_launch<double, 64, false>(n, a, lda, stride, batch, info, s);
}

}  // namespace bl
