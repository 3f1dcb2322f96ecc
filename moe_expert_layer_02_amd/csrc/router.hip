// Router: logits and the two routing families, one wavefront per token.
//
// [Edge0, section 2 "MoE routing"]: softmax-top-k takes an exact softmax over
// the E logits, keeps the k best and renormalises; sigmoid-group scores experts
// with a sigmoid, ranks groups by the sum of their two best scores, keeps the
// best topk_group groups, picks the top k inside them and renormalises the raw
// sigmoid scores with a scale factor.
//
// Lane l of the wavefront owns experts [l*NPL, l*NPL + NPL).  A selection round
// is one wavefront max over 64-bit keys (order-preserving float bits in the high
// word, the complemented expert id in the low word, so equal logits go to the
// lower id).  Group scores are formed in double precision from the float
// logits; expert ranking uses the float logits.
#include "internal.h"

namespace moe355 {
namespace {

__device__ __forceinline__ float key_to_f32(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t make_key(float v, int e) {
    return (static_cast<uint64_t>(f32_order_key(v)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(e));
}

// Top-2 merge of (a1 >= a2) with (b1 >= b2).
__device__ __forceinline__ void top2_merge(double& a1, double& a2, double b1, double b2) {
    double hi = fmax(a1, b1);
    double lo = fmax(fmin(a1, b1), fmax(a2, b2));
    a1 = hi;
    a2 = lo;
}

template <int NPL>
__global__ void __launch_bounds__(256) route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, int kind, int n_group, int topk_group,
                                                    float route_scale, int32_t* __restrict__ ids,
                                                    float* __restrict__ wout) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int t = blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE;
    if (t >= T) return;  // whole wavefront leaves together
    const float* lg = logits + static_cast<int64_t>(t) * E;

    float v[NPL];
    bool valid[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        int e = lane * NPL + i;
        valid[i] = e < E;
        v[i] = valid[i] ? lg[e] : 0.0f;
    }

    bool eligible[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) eligible[i] = valid[i];

    if (kind == MOE355_ROUTE_SIGMOID_GROUP) {
        const int gsize = E / n_group;
        const int lpg = gsize / NPL;  // lanes per group (power of two, checked on the host)
        double s1 = -1.0, s2 = -1.0;  // sigmoid scores are > 0, so -1 is "none"
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
            if (!valid[i]) continue;
            double s = 1.0 / (1.0 + exp(-static_cast<double>(v[i])));
            top2_merge(s1, s2, s, -1.0);
        }
        for (int m = 1; m < lpg; m <<= 1) {
            double b1 = __shfl_xor(s1, m, WAVE);
            double b2 = __shfl_xor(s2, m, WAVE);
            top2_merge(s1, s2, b1, b2);
        }
        const double score = s1 + s2;
        const int my_group = lane / lpg;
        int rank = 0;
        for (int g = 0; g < n_group; ++g) {
            double sg = __shfl(score, g * lpg, WAVE);
            if (sg > score || (sg == score && g < my_group)) ++rank;
        }
        const bool kept = my_group < n_group && rank < topk_group;
#pragma unroll
        for (int i = 0; i < NPL; ++i) eligible[i] = eligible[i] && kept;
    }

    uint64_t key[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) key[i] = eligible[i] ? make_key(v[i], lane * NPL + i) : 0ull;

    int my_e = 0;
    float my_v = 0.0f;
    float vmax = 0.0f;
    for (int r = 0; r < k; ++r) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < NPL; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
        const int e = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best));
        const float val = key_to_f32(static_cast<uint32_t>(best >> 32));
#pragma unroll
        for (int i = 0; i < NPL; ++i)
            if (key[i] == best) key[i] = 0ull;
        if (r == 0) vmax = val;
        if (lane == r) {
            my_e = e;
            my_v = val;
        }
    }

    if (kind == MOE355_ROUTE_SOFTMAX_TOPK) {
        float p = lane < k ? expf(my_v - vmax) : 0.0f;
        float sum = wave_sum_f32(p);
        if (lane < k) {
            ids[static_cast<int64_t>(t) * k + lane] = my_e;
            wout[static_cast<int64_t>(t) * k + lane] = p / sum;
        }
    } else {
        double s = lane < k ? 1.0 / (1.0 + exp(-static_cast<double>(my_v))) : 0.0;
        double sum = s;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, WAVE);
        if (lane < k) {
            ids[static_cast<int64_t>(t) * k + lane] = my_e;
            wout[static_cast<int64_t>(t) * k + lane] =
                static_cast<float>(s / sum * static_cast<double>(route_scale));
        }
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

moe355_status launch_route(const moe355_layer_desc* d, const float* logits, int32_t T,
                           int32_t* ids, float* w, hipStream_t stream) {
    const int E = d->n_experts, k = d->top_k;
    const int npl = (E + WAVE - 1) / WAVE;
    const int blocks = (T + 3) / 4;
    switch (npl) {
#define MOE355_ROUTE_CASE(N)                                                                   \
    case N:                                                                                     \
        route_kernel<N><<<blocks, 256, 0, stream>>>(logits, T, E, k, d->route, d->n_group,     \
                                                    d->topk_group, d->route_scale, ids, w);    \
        break;
        MOE355_ROUTE_CASE(1)
        MOE355_ROUTE_CASE(2)
        MOE355_ROUTE_CASE(3)
        MOE355_ROUTE_CASE(4)
        MOE355_ROUTE_CASE(5)
        MOE355_ROUTE_CASE(6)
        MOE355_ROUTE_CASE(7)
        MOE355_ROUTE_CASE(8)
#undef MOE355_ROUTE_CASE
        default:
            return fail(MOE355_ENOTSUP, "route: E=%d exceeds 512", E);
    }
    return check_launch("route");
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
    const int E = d->n_experts, k = d->top_k;
    MOE355_REQUIRE(E <= 512, MOE355_ENOTSUP, "route: E=%d > 512", E);
    MOE355_REQUIRE(k >= 1 && k <= 32 && k <= E, MOE355_ENOTSUP, "route: k=%d (E=%d)", k, E);
    if (d->route == MOE355_ROUTE_SIGMOID_GROUP) {
        const int npl = (E + WAVE - 1) / WAVE;
        const int gsize = E / d->n_group;
        const int lpg = gsize / npl;
        MOE355_REQUIRE(gsize >= 2 && gsize % npl == 0 && lpg >= 1 && lpg <= WAVE &&
                           (lpg & (lpg - 1)) == 0,
                       MOE355_ENOTSUP, "route: group size %d does not split over lanes (E=%d)",
                       gsize, E);
        MOE355_REQUIRE(d->n_group * gsize == E, MOE355_EINVAL, "route: E=%d not divisible by %d",
                       E, d->n_group);
        MOE355_REQUIRE(k <= d->topk_group * gsize, MOE355_EINVAL,
                       "route: k=%d exceeds the kept groups' %d experts", k,
                       d->topk_group * gsize);
    }
    if (T == 0) return ok();
    return launch_route(d, logits, T, topk_ids, topk_w, stream);
}
