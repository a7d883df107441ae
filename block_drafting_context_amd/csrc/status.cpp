// status.cpp -- status strings and version of libdflash.so (host only).
#include "dflash.h"

extern "C" const char* dflash_status_string(int status) {
    switch (status) {
        case DFLASH_OK: return "ok";
        case DFLASH_ERR_NULL: return "a required pointer is NULL";
        case DFLASH_ERR_SHAPE: return "invalid size or scalar argument";
        case DFLASH_ERR_UNSUPPORTED: return "configuration outside what this build supports";
        case DFLASH_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case DFLASH_ERR_HIP: return "HIP launch failed";
        case DFLASH_ERR_TOO_LARGE: return "needs more scratch than the static array holds";
        default: return "unknown status";
    }
}

extern "C" int dflash_version(void) { return 100; }
