// Full attention layer entry points (placeholder: not yet enabled).
#include "common.h"

extern "C" {

size_t cluster_attn_layer_workspace_size(int, int, int, int, int, int) { return 0; }

ca_status_t cluster_attn_layer_forward(const void *, const void *, const void *, const void *,
                                       const void *, int, int, int, int, int, int, int, int,
                                       float, void *, int32_t *, void *, void *, size_t,
                                       hipStream_t) {
    return CA_ERR_UNSUPPORTED;
}

ca_status_t ca_gemm_bf16(const void *, const void *, int, int, int, void *, hipStream_t) {
    return CA_ERR_UNSUPPORTED;
}

}  // extern "C"
