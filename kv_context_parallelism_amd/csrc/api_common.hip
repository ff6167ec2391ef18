// api_common.hip -- status strings, per-thread error messages, workspace sizing.
#include <stdarg.h>
#include <stdio.h>

#include "internal.hpp"

namespace cpattn {

static thread_local char g_err[512];

cp_status fail(cp_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

void clear_error() { g_err[0] = 0; }

cp_status check_launch(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(CP_E_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return CP_OK;
}

}  // namespace cpattn

extern "C" {

const char *cp_status_str(cp_status s) {
    switch (s) {
    case CP_OK: return "CP_OK";
    case CP_E_INVALID: return "CP_E_INVALID";
    case CP_E_UNSUPPORTED: return "CP_E_UNSUPPORTED";
    case CP_E_WORKSPACE: return "CP_E_WORKSPACE";
    case CP_E_HIP: return "CP_E_HIP";
    }
    return "unknown cp_status";
}

const char *cp_last_error(void) { return cpattn::g_err; }

int cp_abi_version(void) { return CP_ABI_VERSION; }

size_t cp_workspace_bytes(int op, const void *args) {
    if (!args) return (size_t)-1;
    switch (op) {
    case CP_OP_DECODE_GQA: return cpattn::plan_gqa(*static_cast<const cp_gqa_args *>(args)).ws_bytes;
    case CP_OP_DECODE_GQA_MTP:
        return cpattn::plan_gqa_mtp(*static_cast<const cp_gqa_mtp_args *>(args)).ws_bytes;
    case CP_OP_DECODE_MLA: return cpattn::plan_mla(*static_cast<const cp_mla_args *>(args)).ws_bytes;
    case CP_OP_PREFILL: return 0;
    }
    return (size_t)-1;
}

}  // extern "C"
