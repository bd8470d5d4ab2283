// Version and status strings of the C ABI (host only).
#include "../../include/rgc.h"

extern "C" int rgc_abi_version(void) { return RGC_ABI_VERSION; }

extern "C" const char* rgc_status_string(rgc_status_t status) {
  switch (status) {
    case RGC_OK: return "ok";
    case RGC_ERR_NULL: return "a required pointer is NULL";
    case RGC_ERR_SHAPE: return "invalid shape (negative size, r > k or leading dimension < width)";
    case RGC_ERR_UNSUPPORTED: return "unsupported shape (rank, width multiple or size limit)";
    case RGC_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case RGC_ERR_WORKSPACE: return "workspace missing or too small";
    case RGC_ERR_HIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}
