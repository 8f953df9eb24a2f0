// Status strings of the C ABI.
#include "common.h"

extern "C" const char* moe_status_string(moe_status status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_UNSUPPORTED: return "unsupported size";
        case MOE_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}
