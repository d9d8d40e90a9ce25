// Status strings and version of the C ABI.
#include "csa_internal.h"

extern "C" const char* csa_status_string(int status) {
  switch (status) {
    case CSA_OK: return "CSA_OK";
    case CSA_ERR_NULL: return "CSA_ERR_NULL: a required pointer is NULL";
    case CSA_ERR_SHAPE: return "CSA_ERR_SHAPE: unsupported or inconsistent sizes";
    case CSA_ERR_RANGE: return "CSA_ERR_RANGE: positions or block ranges outside the buffers";
    case CSA_ERR_WORKSPACE: return "CSA_ERR_WORKSPACE: workspace missing or too small";
    case CSA_ERR_DTYPE: return "CSA_ERR_DTYPE: unknown dtype code";
    case CSA_ERR_HIP: return "CSA_ERR_HIP: a HIP launch or runtime call failed";
    case CSA_ERR_ALIGN: return "CSA_ERR_ALIGN: pointer or stride alignment";
    case CSA_ERR_SCRATCH:
      return "CSA_ERR_SCRATCH: the call needs more scratch than the static buffer holds";
    default: return "CSA: unknown status";
  }
}

extern "C" int csa_version(void) { return 100; }
