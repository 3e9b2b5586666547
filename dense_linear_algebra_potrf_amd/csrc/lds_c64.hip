// LDS-family kernels for element type cfloat (one translation unit per type so
// the kernels build in parallel).
#include "lds_impl.hpp"

namespace bl {

int lds_max_n_c64() { return lds_detail::last_nb(lds_detail::LdsConfigs<cfloat>::type{}); }

bool lds_geometry_c64(int n, int64_t batch, Geometry& g) {
    return lds_detail::geometry_t<cfloat>(n, batch, g);
}

hipError_t lds_potrf_c64(bool upper, int n, void* A, int64_t lda, int64_t stride, int64_t batch,
                        int32_t* info, hipStream_t s) {
    return lds_detail::potrf_t<cfloat>(upper, n, A, lda, stride, batch, info, s);
}

}  // namespace bl
