// checks.hip -- which build this is, and the record of violated device-data
// preconditions that the build with device checks keeps (host only).
#include "common.hpp"

using namespace dfl;

extern "C" int dflash_device_checks(void) { return DFLASH_DEVICE_CHECKS; }

extern "C" int dflash_violations(uint32_t* word, int clear, void* stream) {
    if (!word) return DFLASH_ERR_NULL;
    *word = 0;
#if DFLASH_DEVICE_CHECKS
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    for (auto reader : {violations_attn, violations_fuse, violations_rows, violations_select}) {
        const int rc = reader(word, clear != 0, st);
        if (rc) return rc;
    }
    return DFLASH_OK;
#else
    (void)clear;
    (void)stream;
    return DFLASH_ERR_UNSUPPORTED;
#endif
}
