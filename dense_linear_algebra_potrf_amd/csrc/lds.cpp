// LDS-family dispatch by element type (host only).
#include "families.hpp"

namespace bl {

#define BL_DECLARE_LDS(suf)                                                                   \
    int lds_max_n_##suf();                                                                    \
    bool lds_geometry_##suf(int n, int64_t batch, Geometry& g);                               \
    hipError_t lds_potrf_##suf(bool upper, int n, void* A, int64_t lda, int64_t stride,       \
                               int64_t batch, int32_t* info, hipStream_t s);
BL_DECLARE_LDS(f32)
BL_DECLARE_LDS(f64)
BL_DECLARE_LDS(c64)
BL_DECLARE_LDS(c128)
#undef BL_DECLARE_LDS

int lds_max_n(DT dt) {
    switch (dt) {
    case DT::F32: return lds_max_n_f32();
    case DT::F64: return lds_max_n_f64();
    case DT::C64: return lds_max_n_c64();
    case DT::C128: return lds_max_n_c128();
    }
    return 0;
}

bool lds_geometry(DT dt, int n, int64_t batch, Geometry& g) {
    switch (dt) {
    case DT::F32: return lds_geometry_f32(n, batch, g);
    case DT::F64: return lds_geometry_f64(n, batch, g);
    case DT::C64: return lds_geometry_c64(n, batch, g);
    case DT::C128: return lds_geometry_c128(n, batch, g);
    }
    return false;
}

hipError_t lds_potrf(DT dt, bool upper, int n, void* A, int64_t lda, int64_t stride,
                     int64_t batch, int32_t* info, hipStream_t s) {
    switch (dt) {
    case DT::F32: return lds_potrf_f32(upper, n, A, lda, stride, batch, info, s);
    case DT::F64: return lds_potrf_f64(upper, n, A, lda, stride, batch, info, s);
    case DT::C64: return lds_potrf_c64(upper, n, A, lda, stride, batch, info, s);
    case DT::C128: return lds_potrf_c128(upper, n, A, lda, stride, batch, info, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace bl
