// ffn_prefill.hip -- expert FFN for large token batches (placeholder).
#include "common.h"

namespace moe {

size_t ffn_prefill_ws_bytes(int d, int f, int E, int T, int k) {
    (void)d; (void)f; (void)E; (void)T; (void)k;
    return 0;
}

hipError_t launch_ffn_prefill(const moe_layer &, const uint16_t *, int, int, const int32_t *,
                              const int32_t *, float *, float *, void *, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace moe
