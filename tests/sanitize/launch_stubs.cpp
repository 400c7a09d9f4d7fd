// Host-only stand-ins for the kernel launchers, for the sanitizer build of
// the C ABI: the validation cases never reach a launch, so each stub reports
// a failure if one is ever called.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>

#include "pdscan_bwd_plan.h"
#include "pdscan_plan.h"
#include "pdscan_sens_plan.h"
#include "pdscan_soft_plan.h"

int g_launches = 0;

namespace pdscan {
static hipError_t stub(const char* name) {
  std::fprintf(stderr, "launcher %s reached in a validation case\n", name);
  ++g_launches;
  return hipErrorInvalidValue;
}
hipError_t launch_select(const Args&, hipStream_t) { return stub("select"); }
hipError_t launch_scan(const Args&, hipStream_t) { return stub("scan"); }
hipError_t launch_gemm_sel(const Args&, hipStream_t) { return stub("gemm_sel"); }
hipError_t launch_gemm_drive(const Args&, float*, hipStream_t) { return stub("gemm_drive"); }
hipError_t launch_fused(const Args&, hipStream_t) { return stub("fused"); }
hipError_t launch_bwd(const BwdArgs&, float*, hipStream_t) { return stub("bwd"); }
hipError_t launch_sens(const SensArgs&, hipStream_t) { return stub("sens"); }
hipError_t launch_soft(const SoftArgs&, hipStream_t) { return stub("soft"); }
hipError_t launch_dict_hardmax(const float*, int32_t*, int, int, hipStream_t) { return stub("dict_hardmax"); }
hipError_t launch_status(const void*, uint32_t*, hipStream_t) { return stub("status"); }
hipError_t noalloc_scratch(void**, size_t*) { return stub("noalloc_scratch"); }
}  // namespace pdscan

extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }
