// Status strings, last HIP error, device properties.
#include "lrc_internal.h"

namespace lrc {

static thread_local int g_last_hip_error = 0;

void set_last_hip_error(hipError_t e) { g_last_hip_error = int(e); }

int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev] = v;
  return v;
}

}  // namespace lrc

extern "C" const char* lrc_status_string(lrc_status s) {
  switch (s) {
    case LRC_OK: return "LRC_OK";
    case LRC_EINVAL: return "LRC_EINVAL: invalid argument";
    case LRC_EDTYPE: return "LRC_EDTYPE: unsupported dtype or flags";
    case LRC_EWORKSPACE: return "LRC_EWORKSPACE: workspace missing or too small";
    case LRC_EHIP: return "LRC_EHIP: HIP runtime error";
    case LRC_ENOTPD: return "LRC_ENOTPD: covariance not positive definite";
    case LRC_ENOCONV: return "LRC_ENOCONV: eigensolver did not converge";
    case LRC_ENONFINITE: return "LRC_ENONFINITE: non-finite value";
  }
  return "unknown lrc_status";
}

extern "C" int lrc_last_hip_error(void) { return lrc::g_last_hip_error; }
