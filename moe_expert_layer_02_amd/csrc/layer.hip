// One decode layer call: route + cache bookkeeping in one workgroup, then the
// expert FFN with fill-through and the combine -- as one launch for a small
// call (the bookkeeping workgroup publishes the plan to the FFN's workgroups
// mid-way), else as two kernels.  Or, split
// so that the bookkeeping leaves the critical path: route + plan, then the FFN
// (hits from slots, misses from the pool) on the caller's stream, while the
// LRU update and the fill copy run on a second stream.
//
// [FT-zh, Method steps]: in decode a single device kernel routes, deduplicates,
// classifies hits, splits the misses by q* and picks K LRU victims; the GPU then
// computes G = H u F while the filled experts are copied into their slots, and
// the partial sums merge exactly -- all inside one captured graph with no host
// involvement.  The tick may live in device memory so a whole decode step can be
// captured once and replayed.
#include "classify_dev.h"

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
    ClassifyParams cp;
    st = classify_setup(c, layer, tick_base, tick_add, nullptr, T * d->top_k, p, lists, &ra,
                        CLASSIFY_FULL, &cp);
    if (st) return st;
    // a small call runs as one launch: the FFN starts once hits and misses are known
    bool launched = false;
    st = decode_layer_small(d, c, pool, layer, cp, x_bf16, T, topk_ids, topk_w, lists, p, out, ws,
                            ws_bytes, stream, &launched);
    if (st || launched) return st;
    st = classify_launch(cp, stream);
    if (st) return st;
    return decode_ffn(d, x_bf16, T, topk_ids, topk_w, c, pool, layer, lists, true, out, ws,
                      ws_bytes, stream);
}

extern "C" moe355_status moe355_route_plan(const moe355_layer_desc* d, const moe355_cache* c,
                                           int32_t layer, const float* logits, int32_t T,
                                           int32_t* topk_ids, float* topk_w,
                                           moe355_classify_out* lists, hipStream_t stream) {
    moe355_status st = check_desc(d);
    if (st) return st;
    st = check_route(d);
    if (st) return st;
    MOE355_REQUIRE(T >= 1 && T * d->top_k <= 256, MOE355_ENOTSUP,
                   "route_plan: T*k=%d outside [1, 256]", T * d->top_k);
    MOE355_REQUIRE(c && logits && topk_ids && topk_w && lists && lists->plan && lists->pairs,
                   MOE355_EINVAL, "route_plan: null pointer");
    MOE355_REQUIRE(c->n_experts == d->n_experts, MOE355_EINVAL,
                   "route_plan: cache holds %d experts per layer, layer has %d", c->n_experts,
                   d->n_experts);
    RouteArgs ra{logits, T, d->top_k, d->route, d->n_group, d->topk_group, d->route_scale,
                 topk_ids, topk_w};
    const moe355_evict_policy none{0, 1, 1};
    return classify_call(c, layer, nullptr, 1, nullptr, T * d->top_k, &none, lists, &ra,
                         CLASSIFY_PLAN, stream);
}

extern "C" moe355_status moe355_evict_fill(const moe355_layer_desc* d, const moe355_cache* c,
                                           const uint8_t* pool, int32_t layer,
                                           const int64_t* tick_base, int64_t tick_add,
                                           const int32_t* topk_ids, int32_t T,
                                           const moe355_evict_policy* p,
                                           moe355_classify_out* lists, hipStream_t stream) {
    moe355_status st = check_desc(d);
    if (st) return st;
    MOE355_REQUIRE(T >= 1 && T * d->top_k <= 256, MOE355_ENOTSUP,
                   "evict_fill: T*k=%d outside [1, 256]", T * d->top_k);
    MOE355_REQUIRE(c && pool && topk_ids && lists && p, MOE355_EINVAL, "evict_fill: null pointer");
    MOE355_REQUIRE(c->n_experts == d->n_experts, MOE355_EINVAL,
                   "evict_fill: cache holds %d experts per layer, layer has %d", c->n_experts,
                   d->n_experts);
    st = classify_call(c, layer, tick_base, tick_add, topk_ids, T * d->top_k, p, lists, nullptr,
                       CLASSIFY_EVICT, stream);
    if (st) return st;
    const int max_fill = p->K < lists->capacity ? p->K : lists->capacity;
    return fill_call(c, pool, layer, lists, max_fill, stream);
}
