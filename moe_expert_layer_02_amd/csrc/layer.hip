// One decode layer call as two kernels: route + cache bookkeeping in one
// workgroup, then the expert FFN with fill-through and the combine.
//
// [FT-zh, Method steps]: in decode a single device kernel routes, deduplicates,
// classifies hits, splits the misses by q* and picks K LRU victims; the GPU then
// computes G = H u F while the filled experts are copied into their slots, and
// the partial sums merge exactly -- all inside one captured graph with no host
// involvement.  The tick may live in device memory so a whole decode step can be
// captured once and replayed.
#include "route_dev.h"

using namespace moe355;

extern "C" moe355_status moe355_decode_layer(const moe355_layer_desc* d, const moe355_cache* c,
                                             const uint8_t* pool, int32_t layer,
                                             const int64_t* tick_base, int64_t tick_add,
                                             const float* logits, const void* x_bf16, int32_t T,
                                             const moe355_evict_policy* p, int32_t* topk_ids,
                                             float* topk_w, moe355_classify_out* lists,
                                             float* out, void* ws, size_t ws_bytes,
                                             hipStream_t stream) {
    moe355_status st = check_desc(d);
    if (st) return st;
    st = check_route(d);
    if (st) return st;
    MOE355_REQUIRE(T >= 1 && T * d->top_k <= 256, MOE355_ENOTSUP,
                   "decode_layer: T*k=%d outside [1, 256]", T * d->top_k);
    MOE355_REQUIRE(c && pool && logits && x_bf16 && topk_ids && topk_w && lists && out,
                   MOE355_EINVAL, "decode_layer: null pointer");
    MOE355_REQUIRE(c->n_experts == d->n_experts, MOE355_EINVAL,
                   "decode_layer: cache holds %d experts per layer, layer has %d", c->n_experts,
                   d->n_experts);
    RouteArgs ra{logits, T, d->top_k, d->route, d->n_group, d->topk_group, d->route_scale,
                 topk_ids, topk_w};
    st = classify_call(c, layer, tick_base, tick_add, nullptr, T * d->top_k, p, lists, &ra, stream);
    if (st) return st;
    return decode_ffn(d, x_bf16, T, topk_ids, topk_w, c, pool, layer, lists, true, out, ws,
                      ws_bytes, stream);
}
