// Dispatch of the split posv route's triangular solves by element type (host
// only).
#include "families.hpp"

namespace bl {

#define BL_DECLARE_POTRS(suf)                                                                  \
    bool potrs_supported_##suf(int n, int nrhs);                                               \
    hipError_t potrs_##suf(bool upper, int n, int nrhs, const void* A, int64_t lda,            \
                           int64_t strideA, void* B, int64_t ldb, int64_t strideB,             \
                           int64_t batch, const int32_t* info, hipStream_t s);
BL_DECLARE_POTRS(f32)
BL_DECLARE_POTRS(f64)
BL_DECLARE_POTRS(c64)
BL_DECLARE_POTRS(c128)
#undef BL_DECLARE_POTRS

bool potrs_supported(DT dt, int n, int nrhs) {
    switch (dt) {
    case DT::F32: return potrs_supported_f32(n, nrhs);
    case DT::F64: return potrs_supported_f64(n, nrhs);
    case DT::C64: return potrs_supported_c64(n, nrhs);
    case DT::C128: return potrs_supported_c128(n, nrhs);
    }
    return false;
}

hipError_t potrs(DT dt, bool upper, int n, int nrhs, const void* A, int64_t lda, int64_t strideA,
                 void* B, int64_t ldb, int64_t strideB, int64_t batch, const int32_t* info,
                 hipStream_t s) {
    switch (dt) {
    case DT::F32: return potrs_f32(upper, n, nrhs, A, lda, strideA, B, ldb, strideB, batch, info, s);
    case DT::F64: return potrs_f64(upper, n, nrhs, A, lda, strideA, B, ldb, strideB, batch, info, s);
    case DT::C64: return potrs_c64(upper, n, nrhs, A, lda, strideA, B, ldb, strideB, batch, info, s);
    case DT::C128: return potrs_c128(upper, n, nrhs, A, lda, strideA, B, ldb, strideB, batch, info, s);
    }
    return hipErrorNotSupported;
}

}  // namespace bl
