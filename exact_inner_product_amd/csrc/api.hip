// api.hip -- status strings, per-thread error state and the profiling hook of libmips.
#include "host.h"

namespace mips {

static thread_local int g_last_hip_error = 0;
static thread_local hipEvent_t g_ev_before = nullptr;
static thread_local hipEvent_t g_ev_after = nullptr;

void set_last_hip_error(hipError_t e) { g_last_hip_error = (int)e; }

void timing_events(hipEvent_t* before, hipEvent_t* after) {
  *before = g_ev_before;
  *after = g_ev_after;
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

}  // namespace mips

extern "C" {

const char* mips_status_string(int status) {
  switch (status) {
    case MIPS_OK: return "ok";
    case MIPS_ERR_INVALID_ARG: return "invalid argument";
    case MIPS_ERR_UNSUPPORTED: return "unsupported size or type";
    case MIPS_ERR_WORKSPACE: return "workspace too small";
    case MIPS_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int mips_last_hip_error(void) { return mips::g_last_hip_error; }

int mips_set_timing_events(void* before, void* after) {
  if (before && after) {
    mips::g_ev_before = (hipEvent_t)before;
    mips::g_ev_after = (hipEvent_t)after;
  } else {
    mips::g_ev_before = nullptr;
    mips::g_ev_after = nullptr;
  }
  return MIPS_OK;
}

}  // extern "C"
