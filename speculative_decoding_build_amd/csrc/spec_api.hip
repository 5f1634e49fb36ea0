// Library-wide entry points that launch nothing.
#include "spec_common.h"

extern "C" int spec_version(void) { return 100; }   // 0.1.0

extern "C" const char *spec_status_string(int status) {
    switch (status) {
        case SPEC_OK: return "ok";
        case SPEC_ERR_NULL: return "a required pointer is NULL";
        case SPEC_ERR_SHAPE: return "sizes inconsistent or out of range";
        case SPEC_ERR_DTYPE: return "unknown dtype code";
        case SPEC_ERR_UNSUPPORTED: return "request outside what this build implements";
        case SPEC_ERR_WORKSPACE: return "workspace missing or too small";
        case SPEC_ERR_HIP: return "HIP launch error";
        default: return "unknown status";
    }
}
