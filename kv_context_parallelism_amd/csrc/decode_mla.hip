// decode_mla.hip -- absorbed-MLA decode partial (placeholder until the MFMA kernel lands).
#include "internal.hpp"

namespace cpattn {
MlaPlan plan_mla(const cp_mla_args &a) {
    (void)a;
    return MlaPlan{0, 1, 0};
}
}  // namespace cpattn

extern "C" cp_status cp_decode_attn_partial_mla(const cp_mla_args *a, void *ws, size_t ws_bytes,
                                                hipStream_t stream) {
    (void)a; (void)ws; (void)ws_bytes; (void)stream;
    return cpattn::fail(CP_E_UNSUPPORTED, "cp_decode_attn_partial_mla: not built yet");
}
