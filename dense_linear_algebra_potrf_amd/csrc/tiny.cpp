// Tiny-family dispatch by element type (host only).
#include "families.hpp"

namespace bl {

#define BL_DECLARE_TINY(suf)                                                                  \
    int tiny_max_n_##suf();                                                                   \
    bool tiny_geometry_##suf(bool upper, int n, int64_t lda, int64_t stride, int64_t batch, Geometry& g);                       \
    bool tiny_layout_ok_##suf(int n, int64_t stride);                                         \
    bool posv_tiny_layout_ok_##suf(int n, int64_t strideA, int64_t strideB);                  \
    int posv_tiny_max_n_##suf();                                                              \
    bool posv_tiny_geometry_##suf(bool upper, int n, int64_t lda, int64_t stride, int64_t batch, Geometry& g);                       \
    hipError_t posv_tiny_##suf(bool upper, int n, int nrhs, void* A, int64_t lda,             \
                               int64_t strideA, void* B, int64_t ldb, int64_t strideB,        \
                               int64_t batch, int32_t* info, hipStream_t s);                  \
    hipError_t tiny_potrf_##suf(bool upper, int n, void* A, int64_t lda, int64_t stride,      \
                                int64_t batch, int32_t* info, hipStream_t s);
BL_DECLARE_TINY(f32)
BL_DECLARE_TINY(f64)
BL_DECLARE_TINY(c64)
BL_DECLARE_TINY(c128)
#undef BL_DECLARE_TINY

int tiny_max_n(DT dt) {
    switch (dt) {
    case DT::F32: return tiny_max_n_f32();
    case DT::F64: return tiny_max_n_f64();
    case DT::C64: return tiny_max_n_c64();
    case DT::C128: return tiny_max_n_c128();
    }
    return 0;
}

bool tiny_layout_ok(DT dt, int n, int64_t stride) {
    switch (dt) {
    case DT::F32: return tiny_layout_ok_f32(n, stride);
    case DT::F64: return tiny_layout_ok_f64(n, stride);
    case DT::C64: return tiny_layout_ok_c64(n, stride);
    case DT::C128: return tiny_layout_ok_c128(n, stride);
    }
    return false;
}

bool tiny_geometry(DT dt, bool upper, int n, int64_t lda, int64_t stride, int64_t batch, Geometry& g) {
    switch (dt) {
    case DT::F32: return tiny_geometry_f32(upper, n, lda, stride, batch, g);
    case DT::F64: return tiny_geometry_f64(upper, n, lda, stride, batch, g);
    case DT::C64: return tiny_geometry_c64(upper, n, lda, stride, batch, g);
    case DT::C128: return tiny_geometry_c128(upper, n, lda, stride, batch, g);
    }
    return false;
}

hipError_t tiny_potrf(DT dt, bool upper, int n, void* A, int64_t lda, int64_t stride,
                      int64_t batch, int32_t* info, hipStream_t s) {
    switch (dt) {
    case DT::F32: return tiny_potrf_f32(upper, n, A, lda, stride, batch, info, s);
    case DT::F64: return tiny_potrf_f64(upper, n, A, lda, stride, batch, info, s);
    case DT::C64: return tiny_potrf_c64(upper, n, A, lda, stride, batch, info, s);
    case DT::C128: return tiny_potrf_c128(upper, n, A, lda, stride, batch, info, s);
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- fused posv
int posv_tiny_max_n(DT dt) {
    switch (dt) {
    case DT::F32: return posv_tiny_max_n_f32();
    case DT::F64: return posv_tiny_max_n_f64();
    case DT::C64: return posv_tiny_max_n_c64();
    case DT::C128: return posv_tiny_max_n_c128();
    }
    return 0;
}
int posv_tiny_max_nrhs() { return 4; }

bool posv_tiny_layout_ok(DT dt, int n, int64_t strideA, int64_t strideB) {
    switch (dt) {
    case DT::F32: return posv_tiny_layout_ok_f32(n, strideA, strideB);
    case DT::F64: return posv_tiny_layout_ok_f64(n, strideA, strideB);
    case DT::C64: return posv_tiny_layout_ok_c64(n, strideA, strideB);
    case DT::C128: return posv_tiny_layout_ok_c128(n, strideA, strideB);
    }
    return false;
}

bool posv_tiny_geometry(DT dt, bool upper, int n, int nrhs, int64_t lda, int64_t stride, int64_t batch, Geometry& g) {
    if (nrhs < 1 || nrhs > posv_tiny_max_nrhs()) return false;
    bool ok = false;
    switch (dt) {
    case DT::F32: ok = posv_tiny_geometry_f32(upper, n, lda, stride, batch, g); break;
    case DT::F64: ok = posv_tiny_geometry_f64(upper, n, lda, stride, batch, g); break;
    case DT::C64: ok = posv_tiny_geometry_c64(upper, n, lda, stride, batch, g); break;
    case DT::C128: ok = posv_tiny_geometry_c128(upper, n, lda, stride, batch, g); break;
    }
    if (!ok) return false;
    g.family = FAM_POSV_TINY;
    return true;
}

hipError_t posv_tiny(DT dt, bool upper, int n, int nrhs, void* A, int64_t lda, int64_t strideA,
                     void* B, int64_t ldb, int64_t strideB, int64_t batch, int32_t* info,
                     hipStream_t s) {
    switch (dt) {
    case DT::F32: return posv_tiny_f32(upper, n, nrhs, A, lda, strideA, B, ldb, strideB, batch, info, s);
    case DT::F64: return posv_tiny_f64(upper, n, nrhs, A, lda, strideA, B, ldb, strideB, batch, info, s);
    case DT::C64: return posv_tiny_c64(upper, n, nrhs, A, lda, strideA, B, ldb, strideB, batch, info, s);
    case DT::C128: return posv_tiny_c128(upper, n, nrhs, A, lda, strideA, B, ldb, strideB, batch, info, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace bl
