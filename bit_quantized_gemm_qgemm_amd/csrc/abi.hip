// Version and status strings of the C ABI.
#include "common.hpp"

extern "C" int32_t qgemm_abi_version(void) { return QGEMM_ABI_VERSION; }

extern "C" const char* qgemm_status_str(int32_t status) {
    switch (status) {
        case QGEMM_OK: return "ok";
        case QGEMM_NULL_PTR: return "null pointer";
        case QGEMM_BAD_SHAPE: return "bad shape";
        case QGEMM_MISALIGNED: return "misaligned pointer";
        case QGEMM_WORKSPACE_TOO_SMALL: return "workspace too small";
        case QGEMM_UNSUPPORTED: return "unsupported shape or option";
        case QGEMM_HIP_ERROR: return "HIP error";
        default: return "unknown status";
    }
}
