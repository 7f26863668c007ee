// Library-wide entry points: ABI version and status strings.
#include "pkv_host.h"

extern "C" int pkv_abi_version(void) { return PKV_ABI_VERSION; }

extern "C" const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_INVALID_ARG: return "PKV_ERR_INVALID_ARG: null pointer, bad size or inconsistent shape";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED: page size, head_dim or dtype combination not built";
    case PKV_ERR_MISALIGNED: return "PKV_ERR_MISALIGNED: a tensor pointer is not 16-byte aligned";
    case PKV_ERR_WORKSPACE_TOO_SMALL: return "PKV_ERR_WORKSPACE_TOO_SMALL: workspace below the queried size";
    case PKV_ERR_HIP: return "PKV_ERR_HIP: a kernel launch failed";
    case PKV_ERR_SCRATCH_TOO_SMALL:
      return "PKV_ERR_SCRATCH_TOO_SMALL: the call needs more than the library's static scratch holds";
    default: return "PKV_ERR_UNKNOWN";
  }
}
