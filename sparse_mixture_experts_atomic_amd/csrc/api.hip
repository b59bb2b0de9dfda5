// Host-only entry points: version, status text, last HIP error, capacity.
#include <math.h>

#include "moe_internal.hpp"

namespace moe {
static thread_local int g_last_hip_error = 0;
void record_hip_error(hipError_t e) { g_last_hip_error = static_cast<int>(e); }
}  // namespace moe

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument (shape, dtype, pointer or k)";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: valid but unimplemented combination";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch failed (see moe_last_hip_error)";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_SCRATCH_LIMIT:
      return "MOE_ERR_SCRATCH_LIMIT: the call needs more scratch than the allocation-free entry point's fixed "
             "MOE_NOALLOC_SCRATCH_BYTES";
    default: return "unknown moe_status";
  }
}

int moe_last_hip_error(void) { return moe::g_last_hip_error; }

// Capacity = round(T * k * cf / E).  Capacity scales with k (a top-2 layer
// gets twice the slots of a top-1 layer at the same factor); the rounding
// mode is selectable (rounding down reproduces 1000 tokens / 8 experts /
// factor 1.25 -> 156).
int moe_capacity(int T, int k, int E, double cf, int round_mode) {
  if (T < 0 || k < 1 || E < 1) return MOE_ERR_INVALID_ARG;
  if (round_mode != MOE_CAP_CEIL && round_mode != MOE_CAP_FLOOR) return MOE_ERR_INVALID_ARG;
  if (!(cf > 0.0)) return -1;
  double v = static_cast<double>(T) * static_cast<double>(k) * cf / static_cast<double>(E);
  double r = round_mode == MOE_CAP_CEIL ? ceil(v) : floor(v);
  if (r > 2147483647.0) return MOE_ERR_INVALID_ARG;
  return static_cast<int>(r);
}

}  // extern "C"
