// C-ABI entry points: argument validation, the size dispatcher, route pins
// and tracing.  Declared in include/batchlas.h.
//
// Validation order and the error/exception mapping follow the BatchLAS
// design_flat_selection page (section on pins: a pin that does not parse or
// cannot run the shape is an error) and the perf_potrf page (section
// "Selection": n >= 1 and batch >= 1, a bad pin is an error; section "posv
// selection": an empty problem is an error).  Everything here runs before
// anything is enqueued, and nothing is written on an error.
#include "../../include/batchlas.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <exception>
#include <mutex>
#include <string>

#include "families.hpp"

namespace {

using bl::DT;
using bl::Geometry;

thread_local std::string g_last_error;

batchlas_status fail(batchlas_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

// ---------------------------------------------------------------- environment snapshot
struct EnvSnapshot {
    int potrf_pin = bl::FAM_AUTO;
    int posv_pin = bl::FAM_AUTO;
    bool potrf_pin_bad = false;
    bool posv_pin_bad = false;
    std::string potrf_pin_text, posv_pin_text;
    bool trace = false;
};

int parse_potrf_pin(const char* s, bool& bad) {
    bad = false;
    if (!s || !*s || !strcmp(s, "auto")) return bl::FAM_AUTO;
    if (!strcmp(s, "tiny")) return bl::FAM_TINY;
    if (!strcmp(s, "lds")) return bl::FAM_LDS;
    if (!strcmp(s, "blocked")) return bl::FAM_BLOCKED;
    bad = true;
    return bl::FAM_AUTO;
}

int parse_posv_pin(const char* s, bool& bad) {
    bad = false;
    if (!s || !*s || !strcmp(s, "auto")) return bl::FAM_AUTO;
    if (!strcmp(s, "tiny") || !strcmp(s, "posv_tiny")) return bl::FAM_POSV_TINY;
    if (!strcmp(s, "split")) return bl::FAM_POSV_SPLIT;
    bad = true;
    return bl::FAM_AUTO;
}

const EnvSnapshot& env() {
    static EnvSnapshot snap;
    static std::once_flag once;
    std::call_once(once, [] {
        const char* p = std::getenv("BATCHLAS_POTRF_ROUTE");
        const char* q = std::getenv("BATCHLAS_POSV_ROUTE");
        const char* t = std::getenv("BATCHLAS_TRACE");
        snap.potrf_pin = parse_potrf_pin(p, snap.potrf_pin_bad);
        snap.posv_pin = parse_posv_pin(q, snap.posv_pin_bad);
        snap.potrf_pin_text = p ? p : "";
        snap.posv_pin_text = q ? q : "";
        snap.trace = t && *t && strcmp(t, "0") != 0;
    });
    return snap;
}

const char* family_name(int f) {
    switch (f) {
    case bl::FAM_AUTO: return "auto";
    case bl::FAM_TINY: return "tiny";
    case bl::FAM_LDS: return "lds";
    case bl::FAM_BLOCKED: return "blocked";
    case bl::FAM_POSV_TINY: return "posv_tiny";
    case bl::FAM_POSV_SPLIT: return "posv_split";
    }
    return "?";
}

const char* dtype_name(DT dt) {
    switch (dt) {
    case DT::F32: return "f32";
    case DT::F64: return "f64";
    case DT::C64: return "c64";
    case DT::C128: return "c128";
    }
    return "?";
}

// ---------------------------------------------------------------- dispatcher thresholds
// Largest order the dispatcher sends to the tiny family, per element type;
// above it the LDS family up to auto_lds_cut, the blocked family beyond.
// Values come from measurements of the families on MI355X.
int auto_tiny_cut(DT dt) {
    switch (dt) {
    // fp32: the 64 x 1 window (184 us against 392 at n=48, b16384), then the wide
    // window: 2.5-3.9x faster than the blocked family at 65..128 (two wavefronts,
    // a row per lane: n=65 b16384 342 us against 1348, n=128 b8192 353 against
    // 899), 1.4-1.5x at 129..192 (tiles: n=129 896 against 1245, n=192 b3640 498
    // against 732); Upper alike
    case DT::F32: return 192;
    // fp64: 64 x 1 (324 us against 438 at n=33, 342 against 2593 at n=64), then
    // the wide window's tiles, 1.3-1.8x faster than the blocked family at 65..128
    // (n=65 b15883 789 us against 1403, n=128 b4096 375 against 503) and slower
    // above (n=144 731 against 578, n=192 553 against 448)
    case DT::F64: return 128;
    // cfloat: the 64 x 1 window beats the LDS family at 33..64; the wide window's
    // tiles beat both other families at every order 65..192 (n=65 b15883 1454 us
    // against 2900 LDS, n=128 b4096 697 against 1963 blocked, n=192 b1820 1026
    // against 1616)
    case DT::C64: return 192;
    // cdouble: 32 x 1 (90-115 us against 321-993 at n=17..32), then the wide
    // tiles at every order 33..192 (n=33 b16384 476 against 597-1020 LDS, n=64
    // b8192 300 against 1694, n=128 b2048 638 against 1153 blocked, n=192 b910
    // 606 against 997)
    case DT::C128: return 192;
    }
    return 0;
}

// ---------------------------------------------------------------- validation
bool mul_ok(int64_t a, int64_t b, int64_t& out) { return !__builtin_mul_overflow(a, b, &out); }

batchlas_status check_common(int dt, int uplo, int64_t n, int64_t nrhs, bool is_posv,
                             int64_t lda, int64_t strideA, int64_t ldb, int64_t strideB,
                             int64_t batch, const void* A, const void* B, bool check_ptrs) {
    if (n < 1) return fail(BATCHLAS_INVALID_VALUE, "n must be >= 1");
    if (n > (int64_t(1) << 24)) return fail(BATCHLAS_INVALID_VALUE, "n is out of range");
    if (is_posv && nrhs < 1) return fail(BATCHLAS_INVALID_VALUE, "nrhs must be >= 1");
    if (is_posv && nrhs > (int64_t(1) << 24)) return fail(BATCHLAS_INVALID_VALUE, "nrhs is out of range");
    if (batch < 1) return fail(BATCHLAS_INVALID_VALUE, "batch must be >= 1");
    if (lda < n) return fail(BATCHLAS_INVALID_VALUE, "lda must be >= n");
    if (is_posv && ldb < n) return fail(BATCHLAS_INVALID_VALUE, "ldb must be >= n");
    int64_t need = 0;
    if (!mul_ok(lda, n, need) || strideA < need)
        return fail(BATCHLAS_INVALID_VALUE, "strideA must be >= lda * n");
    if (is_posv && (!mul_ok(ldb, nrhs, need) || strideB < need))
        return fail(BATCHLAS_INVALID_VALUE, "strideB must be >= ldb * nrhs");
    int64_t total = 0;
    if (!mul_ok(strideA, batch, total) || (is_posv && !mul_ok(strideB, batch, total)))
        return fail(BATCHLAS_INVALID_VALUE, "batch * stride overflows");
    if (check_ptrs && !A) return fail(BATCHLAS_NULL_POINTER, "A is NULL");
    if (check_ptrs && is_posv && !B) return fail(BATCHLAS_NULL_POINTER, "B is NULL");
    if (dt < 0 || dt > 3) return fail(BATCHLAS_INVALID_VALUE, "unknown dtype");
    if (uplo != BATCHLAS_LOWER && uplo != BATCHLAS_UPPER)
        return fail(BATCHLAS_INVALID_VALUE, "uplo must be LOWER or UPPER");
    return BATCHLAS_OK;
}

// ---------------------------------------------------------------- routing
bool family_can_run_potrf(int fam, DT dt, int n, int64_t lda, int64_t stride) {
    switch (fam) {
    case bl::FAM_TINY: return n <= bl::tiny_max_n(dt) && bl::tiny_layout_ok(dt, n, stride);
    case bl::FAM_LDS: return n <= bl::lds_max_n(dt);
    case bl::FAM_BLOCKED: return bl::blocked_supported(dt, n, lda);
    }
    return false;
}

// Largest order the dispatcher sends to the LDS family when the tiny family
// cannot take the shape (a stride beyond its 31-bit offsets); the blocked
// family takes everything above it.  From a sweep of the three
// families on MI355X at orders 48..256 (batches of 16384 or 512 MB, both uplo,
// us per call, LDS against blocked): the real types lose on the LDS family at
// every order it serves above 64 (fp32 n=65 2441 against 1340, n=96 3094
// against 1217; fp64 n=65 2716 against 1404, n=96 1814 against 662), the
// complex types win on it (cfloat n=65 2897 against 5444, n=96 1934 against
// 2572; cdouble n=48 1272 against 3470, n=64 1690 against 1976).
int auto_lds_cut(DT dt) {
    switch (dt) {
    case DT::F32: return 0;
    case DT::F64: return 0;
    case DT::C64: return 96;
    case DT::C128: return 64;
    }
    return 0;
}

int auto_potrf_family(DT dt, int n, int64_t lda, int64_t stride) {
    const bool tiny = family_can_run_potrf(bl::FAM_TINY, dt, n, lda, stride);
    if (tiny && n <= auto_tiny_cut(dt)) return bl::FAM_TINY;
    if (n <= auto_lds_cut(dt) && family_can_run_potrf(bl::FAM_LDS, dt, n, lda, stride))
        return bl::FAM_LDS;
    if (family_can_run_potrf(bl::FAM_BLOCKED, dt, n, lda, stride)) return bl::FAM_BLOCKED;
    if (tiny) return bl::FAM_TINY;
    return bl::FAM_AUTO;
}

batchlas_status route_potrf(int requested, DT dt, bool upper, int n, int64_t lda, int64_t stride,
                            int64_t batch, Geometry& g) {
    int fam = requested;
    if (fam == bl::FAM_AUTO) {
        const EnvSnapshot& e = env();
        if (e.potrf_pin_bad)
            return fail(BATCHLAS_INVALID_VALUE,
                        "BATCHLAS_POTRF_ROUTE='" + e.potrf_pin_text + "' does not parse "
                        "(auto|tiny|lds|blocked)");
        fam = e.potrf_pin;
    }
    if (fam == bl::FAM_AUTO) fam = auto_potrf_family(dt, n, lda, stride);
    if (fam == bl::FAM_AUTO)
        return fail(BATCHLAS_NOT_SUPPORTED, "no potrf family serves this shape");
    if (fam != bl::FAM_TINY && fam != bl::FAM_LDS && fam != bl::FAM_BLOCKED)
        return fail(BATCHLAS_INVALID_VALUE, std::string("family ") + family_name(fam) +
                                                " is not a potrf family");
    if (!family_can_run_potrf(fam, dt, n, lda, stride))
        return fail(BATCHLAS_NOT_SUPPORTED, std::string("potrf family ") + family_name(fam) +
                                                " cannot run " + dtype_name(dt) + " n=" +
                                                std::to_string(n));
    bool ok = false;
    switch (fam) {
    case bl::FAM_TINY: ok = bl::tiny_geometry(dt, upper, n, lda, stride, batch, g); break;
    case bl::FAM_LDS: ok = bl::lds_geometry(dt, n, batch, g); break;
    case bl::FAM_BLOCKED: ok = bl::blocked_geometry(dt, n, batch, g); break;
    }
    if (!ok) return fail(BATCHLAS_INTERNAL, "geometry unavailable for a runnable family");
    return BATCHLAS_OK;
}

batchlas_status route_posv(int requested, DT dt, bool upper, int n, int nrhs, int64_t lda,
                           int64_t strideA, int64_t strideB, int64_t batch, Geometry& g) {
    int fam = requested;
    if (fam == bl::FAM_AUTO) {
        const EnvSnapshot& e = env();
        if (e.posv_pin_bad)
            return fail(BATCHLAS_INVALID_VALUE, "BATCHLAS_POSV_ROUTE='" + e.posv_pin_text +
                                                    "' does not parse (auto|tiny|split)");
        fam = e.posv_pin;
    }
    const bool tiny_ok = n <= bl::posv_tiny_max_n(dt) && nrhs <= bl::posv_tiny_max_nrhs() &&
                         bl::posv_tiny_layout_ok(dt, n, strideA, strideB);
    if (fam == bl::FAM_AUTO) fam = tiny_ok ? bl::FAM_POSV_TINY : bl::FAM_POSV_SPLIT;
    if (fam == bl::FAM_POSV_TINY) {
        if (!tiny_ok)
            return fail(BATCHLAS_NOT_SUPPORTED, "posv_tiny cannot run " + std::string(dtype_name(dt)) +
                                                    " n=" + std::to_string(n) + " nrhs=" +
                                                    std::to_string(nrhs));
        if (!bl::posv_tiny_geometry(dt, upper, n, nrhs, lda, strideA, batch, g))
            return fail(BATCHLAS_INTERNAL, "geometry unavailable for posv_tiny");
        return BATCHLAS_OK;
    }
    if (fam == bl::FAM_POSV_SPLIT) {
        if (!bl::potrs_supported(dt, n, nrhs))
            return fail(BATCHLAS_NOT_SUPPORTED, "the fused two-solve kernel cannot run " +
                                                    std::string(dtype_name(dt)) + " n=" +
                                                    std::to_string(n) + " nrhs=" +
                                                    std::to_string(nrhs));
        Geometry pg;
        batchlas_status st = route_potrf(bl::FAM_AUTO, dt, upper, n, lda, strideA, batch, pg);
        if (st != BATCHLAS_OK) return st;
        g = pg;
        g.family = bl::FAM_POSV_SPLIT;
        return BATCHLAS_OK;
    }
    return fail(BATCHLAS_INVALID_VALUE, std::string("family ") + family_name(fam) +
                                            " is not a posv family");
}

void trace(const char* op, DT dt, int uplo, int64_t n, int64_t nrhs, int64_t batch,
           const Geometry& g) {
    if (!env().trace) return;
    std::fprintf(stderr,
                 "[batchlas] %s %s %s n=%lld nrhs=%lld batch=%lld -> %s P=%d R=%d G=%d "
                 "threads=%d panel=%d grid=%lld lds=%lld\n",
                 op, dtype_name(dt), uplo == BATCHLAS_UPPER ? "U" : "L", (long long)n,
                 (long long)nrhs, (long long)batch, family_name(g.family), g.P, g.R, g.G,
                 g.threads, g.panel, (long long)g.grid, (long long)g.lds);
}

// ---------------------------------------------------------------- device check
// The library carries gfx950 code only; refuse other devices up front.
batchlas_status check_device() {
    static std::atomic<int> state[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return fail(BATCHLAS_HIP_ERROR, "hipGetDevice failed");
    if (dev < 0 || dev >= 64) return fail(BATCHLAS_NOT_SUPPORTED, "device index out of range");
    int s = state[dev].load(std::memory_order_acquire);
    if (s == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return fail(BATCHLAS_HIP_ERROR, "hipGetDeviceProperties failed");
        s = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        state[dev].store(s, std::memory_order_release);
    }
    if (s != 1) return fail(BATCHLAS_NOT_SUPPORTED, "this library is built for gfx950 only");
    return BATCHLAS_OK;
}

batchlas_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return BATCHLAS_OK;
    return fail(BATCHLAS_HIP_ERROR, std::string(what) + ": " + hipGetErrorString(e));
}

batchlas_status do_potrf(int family, int dt_, int uplo, int64_t n, void* A, int64_t lda,
                         int64_t strideA, int64_t batch, int32_t* info, batchlas_stream_t stream) {
    batchlas_status st = check_common(dt_, uplo, n, 0, false, lda, strideA, 0, 0, batch, A,
                                      nullptr, true);
    if (st != BATCHLAS_OK) return st;
    const DT dt = static_cast<DT>(dt_);
    Geometry g;
    st = route_potrf(family, dt, uplo == BATCHLAS_UPPER, int(n), lda, strideA, batch, g);
    if (st != BATCHLAS_OK) return st;
    st = check_device();
    if (st != BATCHLAS_OK) return st;
    trace("potrf", dt, uplo, n, 0, batch, g);
    const bool upper = uplo == BATCHLAS_UPPER;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipErrorInvalidValue;
    switch (g.family) {
    case bl::FAM_TINY: e = bl::tiny_potrf(dt, upper, int(n), A, lda, strideA, batch, info, s); break;
    case bl::FAM_LDS: e = bl::lds_potrf(dt, upper, int(n), A, lda, strideA, batch, info, s); break;
    case bl::FAM_BLOCKED:
        e = bl::blocked_potrf(dt, upper, int(n), A, lda, strideA, batch, info, s);
        break;
    }
    return hip_status(e, "potrf launch");
}

batchlas_status do_posv(int family, int dt_, int uplo, int64_t n, int64_t nrhs, void* A,
                        int64_t lda, int64_t strideA, void* B, int64_t ldb, int64_t strideB,
                        int64_t batch, int32_t* info, batchlas_stream_t stream) {
    batchlas_status st = check_common(dt_, uplo, n, nrhs, true, lda, strideA, ldb, strideB,
                                      batch, A, B, true);
    if (st != BATCHLAS_OK) return st;
    const DT dt = static_cast<DT>(dt_);
    Geometry g;
    st = route_posv(family, dt, uplo == BATCHLAS_UPPER, int(n), int(nrhs), lda, strideA, strideB,
                    batch, g);
    if (st != BATCHLAS_OK) return st;
    st = check_device();
    if (st != BATCHLAS_OK) return st;
    trace("posv", dt, uplo, n, nrhs, batch, g);
    const bool upper = uplo == BATCHLAS_UPPER;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (g.family == bl::FAM_POSV_TINY)
        return hip_status(bl::posv_tiny(dt, upper, int(n), int(nrhs), A, lda, strideA, B, ldb,
                                        strideB, batch, info, s),
                          "posv launch");
    // split route: potrf, then both solves in one launch (failed items keep B;
    // with info NULL the solve reads the failure off the factor's diagonal)
    st = do_potrf(bl::FAM_AUTO, dt_, uplo, n, A, lda, strideA, batch, info, stream);
    if (st != BATCHLAS_OK) return st;
    return hip_status(bl::potrs(dt, upper, int(n), int(nrhs), A, lda, strideA, B, ldb, strideB,
                                batch, info, s),
                      "potrs launch");
}

template <typename F>
batchlas_status guarded(F&& f) {
    try {
        return f();
    } catch (const std::exception& e) {
        return fail(BATCHLAS_INTERNAL, std::string("internal error: ") + e.what());
    } catch (...) {
        return fail(BATCHLAS_INTERNAL, "internal error");
    }
}

}  // namespace

extern "C" {

batchlas_status batchlas_potrf(batchlas_dtype dt, batchlas_uplo uplo, int64_t n, void* A,
                               int64_t lda, int64_t strideA, int64_t batch, int32_t* info,
                               batchlas_stream_t stream) {
    return guarded([&] {
        return do_potrf(bl::FAM_AUTO, dt, uplo, n, A, lda, strideA, batch, info, stream);
    });
}

batchlas_status batchlas_posv(batchlas_dtype dt, batchlas_uplo uplo, int64_t n, int64_t nrhs,
                              void* A, int64_t lda, int64_t strideA, void* B, int64_t ldb,
                              int64_t strideB, int64_t batch, int32_t* info,
                              batchlas_stream_t stream) {
    return guarded([&] {
        return do_posv(bl::FAM_AUTO, dt, uplo, n, nrhs, A, lda, strideA, B, ldb, strideB, batch,
                       info, stream);
    });
}

batchlas_status batchlas_potrf_family(batchlas_family family, batchlas_dtype dt,
                                      batchlas_uplo uplo, int64_t n, void* A, int64_t lda,
                                      int64_t strideA, int64_t batch, int32_t* info,
                                      batchlas_stream_t stream) {
    return guarded([&] {
        if (family < BATCHLAS_FAMILY_AUTO || family > BATCHLAS_FAMILY_POSV_SPLIT)
            return fail(BATCHLAS_INVALID_VALUE, "unknown family");
        return do_potrf(family, dt, uplo, n, A, lda, strideA, batch, info, stream);
    });
}

batchlas_status batchlas_posv_family(batchlas_family family, batchlas_dtype dt,
                                     batchlas_uplo uplo, int64_t n, int64_t nrhs, void* A,
                                     int64_t lda, int64_t strideA, void* B, int64_t ldb,
                                     int64_t strideB, int64_t batch, int32_t* info,
                                     batchlas_stream_t stream) {
    return guarded([&] {
        if (family < BATCHLAS_FAMILY_AUTO || family > BATCHLAS_FAMILY_POSV_SPLIT)
            return fail(BATCHLAS_INVALID_VALUE, "unknown family");
        return do_posv(family, dt, uplo, n, nrhs, A, lda, strideA, B, ldb, strideB, batch, info,
                       stream);
    });
}

#define BL_TYPED_POTRF(name, DTV, PT)                                                       \
    batchlas_status name(batchlas_uplo uplo, int64_t n, PT* A, int64_t lda, int64_t strideA, \
                         int64_t batch, int32_t* info, batchlas_stream_t stream) {           \
        return batchlas_potrf(DTV, uplo, n, A, lda, strideA, batch, info, stream);           \
    }
BL_TYPED_POTRF(batchlas_spotrf, BATCHLAS_F32, float)
BL_TYPED_POTRF(batchlas_dpotrf, BATCHLAS_F64, double)
BL_TYPED_POTRF(batchlas_cpotrf, BATCHLAS_C64, void)
BL_TYPED_POTRF(batchlas_zpotrf, BATCHLAS_C128, void)
#undef BL_TYPED_POTRF

#define BL_TYPED_POSV(name, DTV, PT)                                                          \
    batchlas_status name(batchlas_uplo uplo, int64_t n, int64_t nrhs, PT* A, int64_t lda,     \
                         int64_t strideA, PT* B, int64_t ldb, int64_t strideB, int64_t batch, \
                         int32_t* info, batchlas_stream_t stream) {                           \
        return batchlas_posv(DTV, uplo, n, nrhs, A, lda, strideA, B, ldb, strideB, batch,     \
                             info, stream);                                                   \
    }
BL_TYPED_POSV(batchlas_sposv, BATCHLAS_F32, float)
BL_TYPED_POSV(batchlas_dposv, BATCHLAS_F64, double)
BL_TYPED_POSV(batchlas_cposv, BATCHLAS_C64, void)
BL_TYPED_POSV(batchlas_zposv, BATCHLAS_C128, void)
#undef BL_TYPED_POSV

batchlas_status batchlas_route(batchlas_family family, batchlas_dtype dt, batchlas_uplo uplo,
                               int64_t n, int64_t nrhs, int64_t lda, int64_t strideA,
                               int64_t batch, batchlas_route_info* out) {
    return guarded([&] {
        if (!out) return fail(BATCHLAS_NULL_POINTER, "out is NULL");
        if (family < BATCHLAS_FAMILY_AUTO || family > BATCHLAS_FAMILY_POSV_SPLIT)
            return fail(BATCHLAS_INVALID_VALUE, "unknown family");
        const bool is_posv = nrhs >= 1;
        batchlas_status st = check_common(dt, uplo, n, nrhs, is_posv, lda, strideA,
                                          is_posv ? n : 0, is_posv ? n * nrhs : 0, batch,
                                          nullptr, nullptr, false);
        if (st != BATCHLAS_OK) return st;
        Geometry g;
        const bool upper = uplo == BATCHLAS_UPPER;
        st = is_posv ? route_posv(family, static_cast<DT>(dt), upper, int(n), int(nrhs), lda,
                                  strideA, n * nrhs, batch, g)
                     : route_potrf(family, static_cast<DT>(dt), upper, int(n), lda, strideA,
                                   batch, g);
        if (st != BATCHLAS_OK) return st;
        out->family = g.family;
        out->lanes_per_matrix = g.P;
        out->rows_per_lane = g.R;
        out->matrices_per_wave = g.G;
        out->block_threads = g.threads;
        out->panel = g.panel;
        out->grid = g.grid;
        out->lds_bytes = g.lds;
        return BATCHLAS_OK;
    });
}

const char* batchlas_status_string(batchlas_status s) {
    switch (s) {
    case BATCHLAS_OK: return "ok";
    case BATCHLAS_INVALID_VALUE: return "invalid value";
    case BATCHLAS_NULL_POINTER: return "null pointer";
    case BATCHLAS_NOT_SUPPORTED: return "not supported";
    case BATCHLAS_HIP_ERROR: return "HIP error";
    case BATCHLAS_INTERNAL: return "internal error";
    }
    return "unknown status";
}

const char* batchlas_last_error(void) { return g_last_error.c_str(); }

int32_t batchlas_version(void) { return 100; }

}  // extern "C"
