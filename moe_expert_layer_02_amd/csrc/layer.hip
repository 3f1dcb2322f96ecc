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
#include <mutex>

#include "classify_dev.h"

using namespace moe355;

namespace {

// ---- the allocation-free variant's scratch ----------------------------------
// One decode workspace per GPU in a file-scope device array: the 64 KiB
// synchronisation header plus h for up to STATIC_TKI values of T*k*I (hi and lo
// 16-bit halves).  Host code never passes the array's name to a kernel (on the
// host it is a stand-in, not a device address): each device's address comes
// from hipGetSymbolAddress, once, with that device current.
constexpr size_t STATIC_SYNC = 65536;
constexpr size_t STATIC_TKI = size_t{1} << 20;
constexpr size_t STATIC_BYTES = STATIC_SYNC + 2 * STATIC_TKI * sizeof(uint16_t);
static __device__ __align__(256) uint8_t scratch[STATIC_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch[MAX_DEVICES] = {};

__global__ void clear_words_kernel(uint32_t* w, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) w[i] = 0u;
}

// This device's scratch address; on the first call on a device, look it up and
// clear its synchronisation header with a kernel on `stream` (a fill kernel, not
// a memset node, so that the call stays safe to capture into a graph).
moe355_status device_scratch(hipStream_t stream, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES)
        return fail(MOE355_EHIP, "decode_layer_static: no usable current device (%d)", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(MOE355_EHIP, "decode_layer_static: scratch address on device %d: %s", dev,
                        hipGetErrorString(e));
        clear_words_kernel<<<64, 256, 0, stream>>>(static_cast<uint32_t*>(ptr),
                                                   static_cast<int>(STATIC_SYNC / 4));
        const moe355_status st = check_launch("decode_layer_static: scratch clear");
        if (st) return st;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return MOE355_OK;
}

// The layer call shared by the workspace and the scratch forms.
moe355_status decode_layer_call(const moe355_layer_desc* d, const moe355_cache* c,
                                const uint8_t* pool, int32_t layer, const int64_t* tick_base,
                                int64_t tick_add, const float* logits, const void* x_bf16,
                                int32_t T, const moe355_evict_policy* p, int32_t* topk_ids,
                                float* topk_w, moe355_classify_out* lists, float* out, void* ws,
                                size_t ws_bytes, hipStream_t stream, uint32_t* err);

}  // namespace

extern "C" moe355_status moe355_decode_layer(const moe355_layer_desc* d, const moe355_cache* c,
                                             const uint8_t* pool, int32_t layer,
                                             const int64_t* tick_base, int64_t tick_add,
                                             const float* logits, const void* x_bf16, int32_t T,
                                             const moe355_evict_policy* p, int32_t* topk_ids,
                                             float* topk_w, moe355_classify_out* lists,
                                             float* out, void* ws, size_t ws_bytes,
                                             hipStream_t stream) {
    return decode_layer_call(d, c, pool, layer, tick_base, tick_add, logits, x_bf16, T, p,
                             topk_ids, topk_w, lists, out, ws, ws_bytes, stream, nullptr);
}

extern "C" moe355_status moe355_decode_layer_static(
    const moe355_layer_desc* d, const moe355_cache* c, const uint8_t* pool, int32_t layer,
    const int64_t* tick_base, int64_t tick_add, const float* logits, const void* x_bf16,
    int32_t T, const moe355_evict_policy* p, int32_t* topk_ids, float* topk_w,
    moe355_classify_out* lists, float* out, uint32_t* err_word, hipStream_t stream) {
    moe355_status st = check_desc(d);
    if (st) return st;
    MOE355_REQUIRE(err_word, MOE355_EINVAL, "decode_layer_static: null error word");
    MOE355_REQUIRE(T >= 1 && T * d->top_k <= 256, MOE355_ENOTSUP,
                   "decode_layer_static: T*k=%d outside [1, 256]", T * d->top_k);
    const size_t tki = static_cast<size_t>(T) * d->top_k * d->inter;
    MOE355_REQUIRE(tki <= STATIC_TKI && decode_ws_bytes(d, T) <= STATIC_BYTES, MOE355_ECAPACITY,
                   "decode_layer_static: T*k*I=%zu beyond the fixed scratch's %zu", tki, STATIC_TKI);
    void* ws = nullptr;
    st = device_scratch(stream, &ws);
    if (st) return st;
    return decode_layer_call(d, c, pool, layer, tick_base, tick_add, logits, x_bf16, T, p,
                             topk_ids, topk_w, lists, out, ws, STATIC_BYTES, stream, err_word);
}

namespace {

moe355_status decode_layer_call(const moe355_layer_desc* d, const moe355_cache* c,
                                const uint8_t* pool, int32_t layer, const int64_t* tick_base,
                                int64_t tick_add, const float* logits, const void* x_bf16,
                                int32_t T, const moe355_evict_policy* p, int32_t* topk_ids,
                                float* topk_w, moe355_classify_out* lists, float* out, void* ws,
                                size_t ws_bytes, hipStream_t stream, uint32_t* err) {
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
                            ws_bytes, stream, &launched, err);
    if (st || launched) return st;
    st = classify_launch(cp, stream);
    if (st) return st;
    return decode_ffn(d, x_bf16, T, topk_ids, topk_w, c, pool, layer, lists, true, out, ws,
                      ws_bytes, stream, err);
}

}  // namespace

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
