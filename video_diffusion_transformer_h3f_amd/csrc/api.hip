// api.hip -- version and status strings of the libh3fused C ABI.
#include "../../include/h3fused.h"

extern "C" int h3f_abi_version(void) { return H3F_ABI_VERSION; }

extern "C" const char* h3f_status_string(h3f_status_t status) {
    switch (status) {
        case H3F_OK: return "ok";
        case H3F_ERR_NULL_POINTER: return "null pointer argument";
        case H3F_ERR_BAD_SHAPE: return "invalid shape or size argument";
        case H3F_ERR_BAD_STRIDE: return "invalid stride (not a vector multiple, or rows/heads overlap)";
        case H3F_ERR_MISALIGNED: return "pointer not 16-byte aligned";
        case H3F_ERR_BAD_DTYPE: return "unsupported data type or type combination";
        case H3F_ERR_ALIASING: return "output overlaps another tensor of the call";
        case H3F_ERR_LAUNCH: return "kernel launch failed";
        case H3F_ERR_UNSUPPORTED: return "size or layout outside the supported range";
        case H3F_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case H3F_ERR_BAD_VALUE: return "argument value outside its valid range";
    }
    return "unknown status";
}
