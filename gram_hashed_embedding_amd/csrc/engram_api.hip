// engram_api.hip -- status strings and version of the libengram.so C ABI.
#include "engram_internal.h"

extern "C" const char *engram_status_string(int status) {
  switch (status) {
    case ENGRAM_OK: return "ok";
    case ENGRAM_EINVAL: return "invalid argument";
    case ENGRAM_EALIGN: return "device buffer not 16-byte aligned";
    case ENGRAM_EWORKSPACE: return "workspace missing or too small";
    case ENGRAM_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

extern "C" int engram_abi_version(void) { return ENGRAM_ABI_VERSION; }
