// Prefill expert FFN (grouped GEMM on the matrix cores).
#include "internal.h"

namespace moe355 {
size_t prefill_ws_bytes(const moe355_layer_desc* d, int T) {
    return static_cast<size_t>(T) * d->top_k * d->inter * sizeof(float) + 256;
}
}  // namespace moe355

using namespace moe355;

extern "C" moe355_status moe355_expert_ffn_prefill(const moe355_layer_desc* d, const void* x_bf16,
                                                   int32_t T, const int32_t* topk_ids,
                                                   const float* topk_w, const uint8_t* layer_w,
                                                   const int32_t* perm, const int32_t* offsets,
                                                   float* out, void* ws, size_t ws_bytes,
                                                   hipStream_t stream) {
    (void)x_bf16; (void)T; (void)topk_ids; (void)topk_w; (void)layer_w; (void)perm;
    (void)offsets; (void)out; (void)ws; (void)ws_bytes; (void)stream;
    moe355_status st = check_desc(d);
    if (st) return st;
    return fail(MOE355_ENOTSUP, "expert_ffn_prefill: not built yet");
}
