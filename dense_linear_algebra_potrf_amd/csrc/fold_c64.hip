// Folded window of the tiny family: cfloat, both triangles (two matrices per
// wavefront, a short and a long row per lane; up to order 48 in the 48-row
// window, 49..56 in the 56-row one).
#include "fold_impl.hpp"

namespace bl {

hipError_t fold_potrf_c64(bool upper, int n, cfloat* a, int64_t lda, int64_t stride, int64_t batch,
                          int32_t* info, hipStream_t s) {
    if (n <= 48)
        return upper ? fold_detail::fold_launch<cfloat, 48, true>(n, a, lda, stride, batch, info, s)
                     : fold_detail::fold_launch<cfloat, 48, false>(n, a, lda, stride, batch, info, s);
    if (n <= 56)
        return upper ? fold_detail::fold_launch<cfloat, 56, true>(n, a, lda, stride, batch, info, s)
                     : fold_detail::fold_launch<cfloat, 56, false>(n, a, lda, stride, batch, info, s);
    return upper ? fold_detail::fold_launch<cfloat, 64, true>(n, a, lda, stride, batch, info, s)
                 : fold_detail::fold_launch<cfloat, 64, false>(n, a, lda, stride, batch, info, s);
}

}  // namespace bl
