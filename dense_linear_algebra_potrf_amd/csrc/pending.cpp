// Families that are not built yet: they report that they cannot run anything,
// so the dispatcher never routes to them and a pin returns NOT_SUPPORTED.
#include "families.hpp"

namespace bl {

int potrs_max_nrhs() { return 0; }
bool potrs_supported(DT, int, int) { return false; }
hipError_t potrs(DT, bool, int, int, const void*, int64_t, int64_t, void*, int64_t, int64_t, int64_t,
                 const int32_t*, hipStream_t) { return hipErrorNotSupported; }

}  // namespace bl
