// Folded window of the tiny family: cdouble, Lower, orders 17..32 in the 32-row
// window (16 lanes per matrix, four matrices per wavefront, a short and a long
// row per lane).
#include "fold_impl.hpp"

namespace bl {

hipError_t fold_potrf_c128(bool upper, int n, cdouble* a, int64_t lda, int64_t stride, int64_t batch,
                           int32_t* info, hipStream_t s) {
    if (upper) return hipErrorInvalidValue;
    return fold_detail::fold_launch<cdouble, 32, false>(n, a, lda, stride, batch, info, s);
}

}  // namespace bl
