// Blocked-family dispatch by element type (host only).
#include "families.hpp"

namespace bl {

#define BL_DECLARE_BLOCKED(suf)                                                               \
    bool blocked_supported_##suf(int n, int64_t lda);                                         \
    bool blocked_geometry_##suf(int n, int64_t batch, Geometry& g);                           \
    hipError_t blocked_potrf_##suf(bool upper, int n, void* A, int64_t lda, int64_t stride,   \
                                   int64_t batch, int32_t* info, hipStream_t s);
BL_DECLARE_BLOCKED(f32)
BL_DECLARE_BLOCKED(f64)
BL_DECLARE_BLOCKED(c64)
BL_DECLARE_BLOCKED(c128)
#undef BL_DECLARE_BLOCKED

bool blocked_supported(DT dt, int n, int64_t lda) {
    switch (dt) {
    case DT::F32: return blocked_supported_f32(n, lda);
    case DT::F64: return blocked_supported_f64(n, lda);
    case DT::C64: return blocked_supported_c64(n, lda);
    case DT::C128: return blocked_supported_c128(n, lda);
    default: return false;
    }
}

bool blocked_geometry(DT dt, int n, int64_t batch, Geometry& g) {
    switch (dt) {
    case DT::F32: return blocked_geometry_f32(n, batch, g);
    case DT::F64: return blocked_geometry_f64(n, batch, g);
    case DT::C64: return blocked_geometry_c64(n, batch, g);
    case DT::C128: return blocked_geometry_c128(n, batch, g);
    default: return false;
    }
}

hipError_t blocked_potrf(DT dt, bool upper, int n, void* A, int64_t lda, int64_t stride,
                         int64_t batch, int32_t* info, hipStream_t s) {
    switch (dt) {
    case DT::F32: return blocked_potrf_f32(upper, n, A, lda, stride, batch, info, s);
    case DT::F64: return blocked_potrf_f64(upper, n, A, lda, stride, batch, info, s);
    case DT::C64: return blocked_potrf_c64(upper, n, A, lda, stride, batch, info, s);
    case DT::C128: return blocked_potrf_c128(upper, n, A, lda, stride, batch, info, s);
    default: return hipErrorNotSupported;
    }
}

}  // namespace bl
