// Router entry points: logits x . W_r^T and routing, one wavefront per token.
// The routing arithmetic itself lives in route_dev.h (shared with the fused
// route + classify kernel).
#include "route_dev.h"

namespace moe355 {
namespace {

__global__ void __launch_bounds__(256) route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, int kind, int n_group, int topk_group,
                                                    float route_scale, int32_t* __restrict__ ids,
                                                    float* __restrict__ wout) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int t = blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE;
    if (t >= T) return;  // whole wavefront leaves together
    float w;
    const int e = route_token(logits + static_cast<int64_t>(t) * E, E, k, kind, n_group, topk_group,
                              route_scale, &w);
    if (lane < k) {
        ids[static_cast<int64_t>(t) * k + lane] = e;
        wout[static_cast<int64_t>(t) * k + lane] = w;
    }
}

// logits[t, e] = x[t, :] . w[e, :]; one block per token, one wavefront per expert.
__global__ void __launch_bounds__(256) router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ w, int T,
                                                            int H, int E,
                                                            float* __restrict__ logits) {
    const int t = blockIdx.x;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wv = threadIdx.x / WAVE;
    const uint16_t* xr = x + static_cast<int64_t>(t) * H;
    for (int e = wv; e < E; e += blockDim.x / WAVE) {
        const float* wr = w + static_cast<int64_t>(e) * H;
        float acc = 0.0f;
        for (int h = lane; h < H; h += WAVE) acc = fmaf(bf16_to_f32(xr[h]), wr[h], acc);
        acc = wave_sum_f32(acc);
        if (lane == 0) logits[static_cast<int64_t>(t) * E + e] = acc;
    }
}

}  // namespace

moe355_status check_route(const moe355_layer_desc* d) {
    const int E = d->n_experts, k = d->top_k;
    MOE355_REQUIRE(E <= WAVE * ROUTE_MAX_NPL, MOE355_ENOTSUP, "route: E=%d > %d", E,
                   WAVE * ROUTE_MAX_NPL);
    MOE355_REQUIRE(k >= 1 && k <= 32 && k <= E, MOE355_ENOTSUP, "route: k=%d (E=%d)", k, E);
    if (d->route == MOE355_ROUTE_SIGMOID_GROUP) {
        const int npl = (E + WAVE - 1) / WAVE;
        const int gsize = E / d->n_group;
        const int lpg = gsize / npl;
        MOE355_REQUIRE(d->n_group * gsize == E, MOE355_EINVAL, "route: E=%d not divisible by %d",
                       E, d->n_group);
        MOE355_REQUIRE(gsize >= 2 && gsize % npl == 0 && lpg >= 1 && lpg <= WAVE &&
                           (lpg & (lpg - 1)) == 0,
                       MOE355_ENOTSUP, "route: group size %d does not split over lanes (E=%d)",
                       gsize, E);
        MOE355_REQUIRE(k <= d->topk_group * gsize, MOE355_EINVAL,
                       "route: k=%d exceeds the kept groups' %d experts", k,
                       d->topk_group * gsize);
    }
    return MOE355_OK;
}

}  // namespace moe355

using namespace moe355;

extern "C" moe355_status moe355_router_logits(const moe355_layer_desc* d, const void* x_bf16,
                                              const float* w_router, int32_t T, float* logits,
                                              hipStream_t stream) {
    moe355_status st = check_desc(d);
    if (st) return st;
    MOE355_REQUIRE(T >= 0, MOE355_EINVAL, "router_logits: T=%d", T);
    MOE355_REQUIRE(T == 0 || (x_bf16 && w_router && logits), MOE355_EINVAL,
                   "router_logits: null pointer");
    if (T == 0) return ok();
    router_logits_kernel<<<T, 256, 0, stream>>>(static_cast<const uint16_t*>(x_bf16), w_router, T,
                                                d->hidden, d->n_experts, logits);
    return check_launch("router_logits");
}

extern "C" moe355_status moe355_route(const moe355_layer_desc* d, const float* logits, int32_t T,
                                      int32_t* topk_ids, float* topk_w, hipStream_t stream) {
    moe355_status st = check_desc(d);
    if (st) return st;
    MOE355_REQUIRE(T >= 0, MOE355_EINVAL, "route: T=%d", T);
    MOE355_REQUIRE(T == 0 || (logits && topk_ids && topk_w), MOE355_EINVAL, "route: null pointer");
    st = check_route(d);
    if (st) return st;
    if (T == 0) return ok();
    route_kernel<<<(T + 3) / 4, 256, 0, stream>>>(logits, T, d->n_experts, d->top_k, d->route,
                                                  d->n_group, d->topk_group, d->route_scale,
                                                  topk_ids, topk_w);
    return check_launch("route");
}
