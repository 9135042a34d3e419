// Status strings and version of the libhlr C ABI (host code only).
#include "hlr_common.hpp"

extern "C" const char *hlr_status_string(hlr_status status) {
  switch (status) {
    case HLR_OK: return "ok";
    case HLR_INVALID_ARG: return "invalid argument";
    case HLR_UNSUPPORTED_DIM: return "unsupported dim";
    case HLR_MISALIGNED: return "misaligned pointer";
    case HLR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case HLR_HIP_ERROR: return "HIP launch error";
    default: return "unknown status";
  }
}

extern "C" int32_t hlr_version(void) { return 103; }
