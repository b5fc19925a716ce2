// Status strings and ABI version of the wedlm library.
#include "common.hpp"

extern "C" const char* wedlm_status_string(int status) {
  switch (status) {
    case WEDLM_OK: return "ok";
    case WEDLM_ERR_INVALID: return "invalid argument";
    case WEDLM_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case WEDLM_ERR_WORKSPACE: return "workspace missing or too small";
    case WEDLM_ERR_HIP: return "HIP launch error";
    case WEDLM_ERR_SCRATCH_LIMIT:
      return "sizes need more than the library's fixed scratch (use the workspace form)";
    default: return "unknown status";
  }
}

extern "C" int wedlm_abi_version(void) { return (1 << 16) | 8; }
