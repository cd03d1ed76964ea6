// api.cpp -- status strings and ABI version of libspecverify.
#include "spec_verify.h"

extern "C" const char* spec_status_string(int code) {
    switch (code) {
        case SPEC_OK: return "ok";
        case SPEC_ERR_INVALID_ARG: return "invalid argument";
        case SPEC_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case SPEC_ERR_HIP: return "HIP launch or runtime error";
        default: return "unknown status";
    }
}

extern "C" int spec_abi_version(void) { return SPEC_VERIFY_ABI_VERSION; }
