// prefill.hip -- PCP causal prefill (placeholder until the MFMA kernel lands).
#include "internal.hpp"

extern "C" cp_status pcp_prefill_attn_causal(const cp_prefill_args *a, void *ws, size_t ws_bytes,
                                             hipStream_t stream) {
    (void)a; (void)ws; (void)ws_bytes; (void)stream;
    return cpattn::fail(CP_E_UNSUPPORTED, "pcp_prefill_attn_causal: not built yet");
}
