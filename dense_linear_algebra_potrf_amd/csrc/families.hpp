// Internal interface between the C-ABI layer (api.cpp) and the kernel
// families.  Every family exposes: can it run a shape, the launch geometry it
// would use, and the enqueue itself.  Geometry and launch come from the same
// configuration tables, so a route query always describes what runs.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.hpp"

namespace bl {

enum Family : int {
    FAM_AUTO = 0,
    FAM_TINY = 1,
    FAM_LDS = 2,
    FAM_BLOCKED = 3,
    FAM_POSV_TINY = 4,
    FAM_POSV_SPLIT = 5,
};

struct Geometry {
    int family = 0;
    int P = 0, R = 0, G = 0;   // tiny / posv: lanes per matrix, rows per lane, matrices per wave
    int threads = 0;           // threads per workgroup of the main kernel
    int panel = 0;             // lds / blocked: panel width
    int64_t grid = 0;          // workgroups of the main kernel (first launch)
    int64_t lds = 0;           // LDS bytes per workgroup of the main kernel
};

// --- tiny: registers, P lanes x R rows per matrix, 64/P matrices per wavefront
int tiny_max_n(DT dt);
bool tiny_layout_ok(DT dt, int n, int64_t stride);   // byte offsets of a wave fit in 31 bits
bool tiny_geometry(DT dt, bool upper, int n, int64_t lda, int64_t stride, int64_t batch, Geometry& g);
hipError_t tiny_potrf(DT dt, bool upper, int n, void* A, int64_t lda, int64_t stride,
                      int64_t batch, int32_t* info, hipStream_t s);

// --- posv tiny: factor + both solves in registers
int posv_tiny_max_n(DT dt);
int posv_tiny_max_nrhs();
bool posv_tiny_layout_ok(DT dt, int n, int64_t strideA, int64_t strideB);
bool posv_tiny_geometry(DT dt, bool upper, int n, int nrhs, int64_t lda, int64_t stride, int64_t batch, Geometry& g);
hipError_t posv_tiny(DT dt, bool upper, int n, int nrhs, void* A, int64_t lda, int64_t strideA,
                     void* B, int64_t ldb, int64_t strideB, int64_t batch, int32_t* info,
                     hipStream_t s);

// --- lds: one workgroup per matrix, matrix staged in LDS
int lds_max_n(DT dt);
bool lds_geometry(DT dt, int n, int64_t batch, Geometry& g);
hipError_t lds_potrf(DT dt, bool upper, int n, void* A, int64_t lda, int64_t stride,
                     int64_t batch, int32_t* info, hipStream_t s);

// --- blocked: panel kernel + MFMA trailing update
bool blocked_supported(DT dt, int n, int64_t lda);   // byte offsets of a matrix fit in 31 bits
bool blocked_geometry(DT dt, int n, int64_t batch, Geometry& g);
hipError_t blocked_potrf(DT dt, bool upper, int n, void* A, int64_t lda, int64_t stride,
                         int64_t batch, int32_t* info, hipStream_t s);

// --- the two triangular solves with an already factored A (posv split route)
bool potrs_supported(DT dt, int n, int nrhs);
hipError_t potrs(DT dt, bool upper, int n, int nrhs, const void* A, int64_t lda,
                 int64_t strideA, void* B, int64_t ldb, int64_t strideB, int64_t batch,
                 const int32_t* info, hipStream_t s);

}  // namespace bl
