// Whole-layer double-buffered prefill over consecutive MoE layers.
//
// [FT-zh, Core method / Method steps: in prefill, two whole-layer buffers --
// while the GPU computes layer l from one, a transfer stream pours layer l+1's
// experts over PCIe into the other, then they swap; loading the whole layer
// lets the transfer start before the routing is known; FT-zh, Results: without
// the second buffer prefill loses 19-26 %.  FT-en, System Architecture: the
// buffer A / buffer B ping-pong.]
//
// The expert pool sits in pinned host memory in the device layout; each
// layer's E * S bytes go to a device buffer by one DMA copy on the caller's
// copy stream, so the matrix cores never wait on the copy engine and vice
// versa.  Per layer l with buffer b (l % 2, or 0 with one buffer):
//   copy stream: wait until the last compute that read buffer b is done,
//                copy layer l into it, record "b loaded";
//   compute stream: wait for "b loaded", route, permute, expert FFN, record
//                "b free".
// With two buffers the copy of layer l+1 runs while layer l computes; with
// one, every copy waits for the previous layer's compute (the ablation).
#include "internal.h"

namespace moe355 {
size_t permute_ws_bytes(int E, int T, int k);
size_t prefill_ws_bytes(const moe355_layer_desc* d, int T);
}  // namespace moe355

using namespace moe355;

namespace {

struct Events {
    hipEvent_t loaded[2] = {nullptr, nullptr};
    hipEvent_t freed[2] = {nullptr, nullptr};
    ~Events() {   // destruction is deferred by the runtime until recorded work completes
        for (int b = 0; b < 2; ++b) {
            if (loaded[b]) (void)hipEventDestroy(loaded[b]);
            if (freed[b]) (void)hipEventDestroy(freed[b]);
        }
    }
};

}  // namespace

extern "C" moe355_status moe355_prefill_layers(
    const moe355_layer_desc* d, int32_t n_layers, int32_t T, const uint8_t* host_pool,
    uint8_t* buf0, uint8_t* buf1, const float* const* logits, const void* const* x,
    float* const* out, int32_t* topk_ids, float* topk_w, int32_t* perm, int32_t* offsets,
    void* ws, size_t ws_bytes, void* perm_ws, size_t perm_ws_bytes, int32_t double_buffer,
    hipStream_t stream, hipStream_t copy_stream) {
    moe355_status st = check_desc(d);
    if (st) return st;
    MOE355_REQUIRE(n_layers >= 1 && T >= 1, MOE355_EINVAL, "prefill_layers: n_layers=%d T=%d",
                   n_layers, T);
    MOE355_REQUIRE(host_pool && buf0 && (buf1 || !double_buffer) && logits && x && out && topk_ids &&
                       topk_w && perm && offsets && ws && perm_ws,
                   MOE355_EINVAL, "prefill_layers: null pointer");
    MOE355_REQUIRE(stream != copy_stream, MOE355_EINVAL,
                   "prefill_layers: the copy stream must differ from the compute stream");
    for (int l = 0; l < n_layers; ++l)
        MOE355_REQUIRE(logits[l] && x[l] && out[l], MOE355_EINVAL, "prefill_layers: null layer %d input",
                       l);
    hipPointerAttribute_t attr;
    MOE355_REQUIRE(hipPointerGetAttributes(&attr, host_pool) == hipSuccess &&
                       attr.type == hipMemoryTypeHost,
                   MOE355_EINVAL, "prefill_layers: host_pool is not pinned host memory");
    MOE355_REQUIRE(ws_bytes >= prefill_ws_bytes(d, T) &&
                       perm_ws_bytes >= permute_ws_bytes(d->n_experts, T, d->top_k),
                   MOE355_ECAPACITY, "prefill_layers: workspace too small");
    ExpertLayout L;
    expert_layout(d, &L);
    const size_t layer_bytes = static_cast<size_t>(L.bytes) * d->n_experts;
    uint8_t* bufs[2] = {buf0, double_buffer ? buf1 : buf0};
    Events ev;
    for (int b = 0; b < 2; ++b)
        if (hipEventCreateWithFlags(&ev.loaded[b], hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&ev.freed[b], hipEventDisableTiming) != hipSuccess)
            return fail(MOE355_EHIP, "prefill_layers: event creation failed");
    for (int l = 0; l < n_layers; ++l) {
        const int b = double_buffer ? (l & 1) : 0;
        // copy stream: the buffer is free once its last reader is done (an
        // event never recorded is complete)
        if (l >= (double_buffer ? 2 : 1) &&
            hipStreamWaitEvent(copy_stream, ev.freed[b], 0) != hipSuccess)
            return fail(MOE355_EHIP, "prefill_layers: wait on layer %d's buffer", l);
        if (hipMemcpyAsync(bufs[b], host_pool + static_cast<size_t>(l) * layer_bytes, layer_bytes,
                           hipMemcpyHostToDevice, copy_stream) != hipSuccess ||
            hipEventRecord(ev.loaded[b], copy_stream) != hipSuccess)
            return fail(MOE355_EHIP, "prefill_layers: copy of layer %d", l);
        // compute stream
        if (hipStreamWaitEvent(stream, ev.loaded[b], 0) != hipSuccess)
            return fail(MOE355_EHIP, "prefill_layers: wait for layer %d's experts", l);
        st = moe355_route(d, logits[l], T, topk_ids, topk_w, stream);
        if (st) return st;
        st = moe355_permute(d, topk_ids, T, perm, offsets, perm_ws, perm_ws_bytes, stream);
        if (st) return st;
        st = moe355_expert_ffn_prefill(d, x[l], T, topk_ids, topk_w, bufs[b], perm, offsets, out[l],
                                       ws, ws_bytes, stream);
        if (st) return st;
        if (hipEventRecord(ev.freed[b], stream) != hipSuccess)
            return fail(MOE355_EHIP, "prefill_layers: record layer %d", l);
    }
    return ok();
}
