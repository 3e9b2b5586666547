// Shared device/host helpers for the batched potrf / posv kernels (gfx950).
//
// Element types are plain structs: complex numbers are interleaved (re, im)
// pairs and every complex product is written out as real multiply-adds (the
// BatchLAS perf_level3 page, section on register-tiled kernels, records that a
// library complex multiply lowers to a slow runtime call and that accumulator
// arrays must stay in registers).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <tuple>
#include <type_traits>
#include <utility>

namespace bl {

struct cfloat { float re, im; };
struct cdouble { double re, im; };

enum class DT : int { F32 = 0, F64 = 1, C64 = 2, C128 = 3 };

template <typename T> struct Traits;
template <> struct Traits<float>   { using R = float;  static constexpr bool cplx = false; static constexpr DT dt = DT::F32; };
template <> struct Traits<double>  { using R = double; static constexpr bool cplx = false; static constexpr DT dt = DT::F64; };
template <> struct Traits<cfloat>  { using R = float;  static constexpr bool cplx = true;  static constexpr DT dt = DT::C64; };
template <> struct Traits<cdouble> { using R = double; static constexpr bool cplx = true;  static constexpr DT dt = DT::C128; };

inline int elem_bytes(DT dt) {
    switch (dt) {
    case DT::F32: return 4;
    case DT::F64: return 8;
    case DT::C64: return 8;
    case DT::C128: return 16;
    }
    return 0;
}

// ---------------------------------------------------------------- scalars
template <typename T> __device__ __forceinline__ T zero() { return T{}; }
template <typename T> __device__ __forceinline__ T one() {
    if constexpr (Traits<T>::cplx) return T{1, 0};
    else return T(1);
}
template <typename T> __device__ __forceinline__ typename Traits<T>::R re(const T& x) {
    if constexpr (Traits<T>::cplx) return x.re;
    else return x;
}
template <typename T> __device__ __forceinline__ T conj(const T& x) {
    if constexpr (Traits<T>::cplx) return T{x.re, -x.im};
    else return x;
}
template <typename T> __device__ __forceinline__ T from_real(typename Traits<T>::R v) {
    if constexpr (Traits<T>::cplx) return T{v, 0};
    else return v;
}
// Real diagonal value whose conjugate has imaginary part +0 (Upper stores conj).
template <typename T> __device__ __forceinline__ T diag_value(typename Traits<T>::R v, bool conj_on_store) {
    using R = typename Traits<T>::R;
    if constexpr (Traits<T>::cplx) return T{v, conj_on_store ? R(-0.0) : R(0.0)};
    else return v;
}
template <typename T> __device__ __forceinline__ T scale(const T& x, typename Traits<T>::R s) {
    if constexpr (Traits<T>::cplx) return T{x.re * s, x.im * s};
    else return x * s;
}
template <typename T> __device__ __forceinline__ T select(bool c, const T& a, const T& b) {
    // component-wise select: keeps aggregates in registers
    if constexpr (Traits<T>::cplx) return T{c ? a.re : b.re, c ? a.im : b.im};
    else return c ? a : b;
}
// Fused multiply-add in the element's own precision (__builtin_fma is the
// double-precision builtin; float needs __builtin_fmaf).
__device__ __forceinline__ float fmadd(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double fmadd(double a, double b, double c) { return __builtin_fma(a, b, c); }

// acc -= t * conj(c)
template <typename T> __device__ __forceinline__ void sub_mul_conj(T& acc, const T& t, const T& c) {
    if constexpr (Traits<T>::cplx) {
        acc.re = fmadd(-t.re, c.re, fmadd(-t.im, c.im, acc.re));
        acc.im = fmadd(-t.im, c.re, fmadd(t.re, c.im, acc.im));
    } else {
        acc = fmadd(-t, c, acc);
    }
}
// acc -= t * c
template <typename T> __device__ __forceinline__ void sub_mul(T& acc, const T& t, const T& c) {
    if constexpr (Traits<T>::cplx) {
        acc.re = fmadd(-t.re, c.re, fmadd(t.im, c.im, acc.re));
        acc.im = fmadd(-t.re, c.im, fmadd(-t.im, c.re, acc.im));
    } else {
        acc = fmadd(-t, c, acc);
    }
}
// acc -= conj(t) * c
template <typename T> __device__ __forceinline__ void sub_conj_mul(T& acc, const T& t, const T& c) {
    if constexpr (Traits<T>::cplx) {
        acc.re = fmadd(-t.re, c.re, fmadd(-t.im, c.im, acc.re));
        acc.im = fmadd(-t.re, c.im, fmadd(t.im, c.re, acc.im));
    } else {
        acc = fmadd(-t, c, acc);
    }
}

// Reciprocal, reciprocal square root and square root of a positive pivot.
// float: the hardware approximations (about 1 ulp), well inside the 1e-4
// parity tolerance.  double: the hardware approximations refined by two Newton
// steps each, which brings them to within a few ulp (far inside the 1e-11
// tolerance) at a fraction of the latency of correctly rounded division and
// square root.  Non-positive pivots give NaN or infinity, as they should: such
// a matrix has already failed.
__device__ __forceinline__ float pivot_rcp(float d) { return __builtin_amdgcn_rcpf(d); }
__device__ __forceinline__ float pivot_rsq(float d) { return __builtin_amdgcn_rsqf(d); }
__device__ __forceinline__ float pivot_sqrt(float d) { return __builtin_amdgcn_sqrtf(d); }
__device__ __forceinline__ void pivot_sqrt_rsq(float d, float& sq, float& rsq) {
    sq = __builtin_amdgcn_sqrtf(d);
    rsq = __builtin_amdgcn_rsqf(d);
}
// 1/d: r <- r + r (1 - d r), twice.
__device__ __forceinline__ double pivot_rcp(double d) {
    double r = __builtin_amdgcn_rcp(d);
    r = __builtin_fma(r, __builtin_fma(-d, r, 1.0), r);
    r = __builtin_fma(r, __builtin_fma(-d, r, 1.0), r);
    return r;
}
// sqrt(d) and 1/sqrt(d) together: from y ~ 1/sqrt(d), g = d y ~ sqrt(d) and
// h = y / 2; each step takes the residual e = 1/2 - g h and sets g += g e,
// h += h e (both converge quadratically).
__device__ __forceinline__ void pivot_sqrt_rsq(double d, double& sq, double& rsq) {
    const double y = __builtin_amdgcn_rsq(d);
    double g = d * y, h = 0.5 * y;
    double e = __builtin_fma(-g, h, 0.5);
    g = __builtin_fma(g, e, g);
    h = __builtin_fma(h, e, h);
    e = __builtin_fma(-g, h, 0.5);
    g = __builtin_fma(g, e, g);
    h = __builtin_fma(h, e, h);
    sq = g;
    rsq = 2.0 * h;
}
__device__ __forceinline__ double pivot_sqrt(double d) { double s, r; pivot_sqrt_rsq(d, s, r); return s; }
__device__ __forceinline__ double pivot_rsq(double d) { double s, r; pivot_sqrt_rsq(d, s, r); return r; }

// All three terms of a pivot, 1/d, 1/sqrt(d) and sqrt(d), from one reciprocal
// square root rs: 1/d = rs rs and sqrt(d) = d rs.  The hardware reciprocal,
// square root and reciprocal square root each issue at a quarter of the
// vector rate, so one of them in place of three shortens every column step.
// float: rs within about 1 ulp, so each term is within a few ulp.  double:
// rs and sqrt(d) from the refined pair above.  A pivot that is not > 0 gives
// NaN or infinity in some term, as it should: that matrix has already failed.
__device__ __forceinline__ void pivot_terms(float d, float& inv, float& rs, float& sq) {
    rs = __builtin_amdgcn_rsqf(d);
    inv = rs * rs;
    sq = d * rs;
}
__device__ __forceinline__ void pivot_terms(double d, double& inv, double& rs, double& sq) {
    pivot_sqrt_rsq(d, sq, rs);
    inv = rs * rs;
}

// ---------------------------------------------------------------- row broadcast multiply-add
// acc += s * x, where x is `col` as held by lane N of this lane's row of 16
// lanes: the DPP row broadcast (row_newbcast, also defined for 64-bit operands)
// is applied to the multiply-add's first operand, so a value spread over 16 lanes feeds 16 updates of every lane
// with no extra instruction.  A DPP read of a register written by a vector ALU
// instruction needs two wait states first; FIRST (the first use of a freshly
// loaded `col`) adds them, in case the compiler copies `col` with a vector move.
template <int N, bool FIRST>
__device__ __forceinline__ void fma_bcast16(float& acc, float s, float col) {
    static_assert(N >= 0 && N < 16, "lane within a row of 16");
    if constexpr (FIRST)
        asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                     : "+v"(acc) : "v"(col), "v"(s), "i"(N));
    else
        asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                     : "+v"(acc) : "v"(col), "v"(s), "i"(N));
}

template <int N, bool FIRST>
__device__ __forceinline__ void fma_bcast16(double& acc, double s, double col) {
    static_assert(N >= 0 && N < 16, "lane within a row of 16");
    if constexpr (FIRST)
        asm volatile("s_nop 1\n\tv_fmac_f64_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                     : "+v"(acc) : "v"(col), "v"(s), "i"(N));
    else
        asm volatile("v_fmac_f64_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                     : "+v"(acc) : "v"(col), "v"(s), "i"(N));
}

// ---------------------------------------------------------------- compile-time loops
template <int V> using ic = std::integral_constant<int, V>;

template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(ic<B>{});
        static_for<B + 1, E>(f);
    }
}

template <int B, int E, typename F>
__device__ __forceinline__ void static_for_down(F&& f) {   // E-1 down to B
    if constexpr (B < E) {
        f(ic<E - 1>{});
        static_for_down<B, E - 1>(f);
    }
}

constexpr int cmin(int a, int b) { return a < b ? a : b; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- LDS element access
// Elements are stored as D = sizeof(T)/4 consecutive dwords.
template <typename T> constexpr int words() { return int(sizeof(T) / 4); }

template <typename T>
__device__ __forceinline__ void lds_put(uint32_t* base, int idx, const T& v) {
    *reinterpret_cast<T*>(base + idx * words<T>()) = v;
}
template <typename T>
__device__ __forceinline__ T lds_get(const uint32_t* base, int idx) {
    return *reinterpret_cast<const T*>(base + idx * words<T>());
}
template <typename T>
__device__ __forceinline__ T from_words(const uint32_t* w) {
    T v;
    __builtin_memcpy(&v, w, sizeof(T));
    return v;
}

// Ordering of LDS traffic between lanes of one wavefront: LDS instructions of a
// wave execute in order, so only the compiler has to be kept from reordering.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- buffer memory access
// Raw buffer loads/stores with a 32-bit byte offset from a wave-uniform base.
// An offset at or above 2^31 is outside the descriptor's range: the load
// returns zero and the store is dropped, without touching memory.  This gives
// branch-free predication that never reads or writes masked elements.
constexpr uint32_t kBufOOB = 0x80000000u;
constexpr int kBufFlags = 0x00020000;   // gfx9-family descriptor word 3 (raw, dword data)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, kBufFlags);
}
// soff is a wave-uniform byte offset (a scalar register) added to off; only off
// takes part in the range check, so a masked off stays out of range.
template <typename T>
__device__ __forceinline__ T buf_load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
    if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0));
    } else if constexpr (sizeof(T) == 8) {
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0));
    } else {
        static_assert(sizeof(T) == 16, "element size");
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
    }
}

template <typename T>
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, uint32_t off, const T& v,
                                          uint32_t soff = 0) {
    if constexpr (sizeof(T) == 4) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, soff, 0);
    } else if constexpr (sizeof(T) == 8) {
        using V = uint32_t __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(V, v), r, off, soff, 0);
    } else {
        using V = uint32_t __attribute__((ext_vector_type(4)));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(V, v), r, off, soff, 0);
    }
}

// ---------------------------------------------------------------- host launch helper
namespace detail {
template <typename Tuple, size_t... I>
inline hipError_t launch_tuple(const void* fn, dim3 g, dim3 b, size_t shm, hipStream_t s, Tuple& t,
                               std::index_sequence<I...>) {
    void* args[] = {static_cast<void*>(&std::get<I>(t))..., nullptr};
    return hipLaunchKernel(fn, g, b, args, shm, s);
}
}  // namespace detail

// Launch a __global__ function and return the launch's own error code.
template <typename... KArgs, typename... Args>
inline hipError_t launch(void (*fn)(KArgs...), dim3 grid, dim3 block, size_t shm, hipStream_t s,
                         Args... args) {
    std::tuple<KArgs...> t(static_cast<KArgs>(args)...);
    return detail::launch_tuple(reinterpret_cast<const void*>(fn), grid, block, shm, s, t,
                                std::index_sequence_for<KArgs...>{});
}

}  // namespace bl
