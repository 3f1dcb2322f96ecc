// Wavefront-level router shared by the route kernel and the fused
// route + classify kernel (included by both translation units).
//
// [Edge0, section 2 "MoE routing"]: softmax-top-k takes an exact softmax over
// the E logits, keeps the k best and renormalises; sigmoid-group scores experts
// with a sigmoid, ranks groups by the sum of their two best scores, keeps the
// best topk_group groups, picks the top k inside them and renormalises the raw
// sigmoid scores with a scale factor.
//
// Lane l owns experts [l*npl, l*npl + npl), npl = ceil(E / 64) <= 8.  A
// selection round is one wavefront max over 64-bit keys (order-preserving float
// bits in the high word, the complemented expert id in the low word, so equal
// logits go to the lower id).  Group scores are formed in double precision from
// the float logits; expert ranking uses the float logits.
#pragma once

#include "internal.h"

namespace moe355 {

constexpr int ROUTE_MAX_NPL = 8;

__device__ __forceinline__ float route_key_to_f32(uint32_t k) {
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t route_key(float v, int e) {
    return (static_cast<uint64_t>(f32_order_key(v)) << 32) |
           (0xFFFFFFFFu - static_cast<uint32_t>(e));
}

// Top-2 merge of (a1 >= a2) with (b1 >= b2).
__device__ __forceinline__ void top2_merge(double& a1, double& a2, double b1, double b2) {
    const double hi = fmax(a1, b1);
    const double lo = fmax(fmin(a1, b1), fmax(a2, b2));
    a1 = hi;
    a2 = lo;
}

// Route one token with one wavefront.  Lane j < k receives the j-th selected
// expert and its weight; the return value is that expert id (meaningful for
// lanes < k only).
__device__ __forceinline__ int route_token(const float* __restrict__ lg, int E, int k, int kind,
                                           int n_group, int topk_group, float route_scale,
                                           float* w_out) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int npl = (E + WAVE - 1) / WAVE;
    float v[ROUTE_MAX_NPL];
    bool eligible[ROUTE_MAX_NPL];
#pragma unroll
    for (int i = 0; i < ROUTE_MAX_NPL; ++i) {
        const int e = lane * npl + i;
        eligible[i] = i < npl && e < E;
        v[i] = eligible[i] ? lg[e] : 0.0f;
    }

    if (kind == MOE355_ROUTE_SIGMOID_GROUP) {
        const int gsize = E / n_group;
        const int lpg = gsize / npl;  // lanes per group (power of two, checked on the host)
        double s1 = -1.0, s2 = -1.0;  // sigmoid scores are > 0, so -1 is "none"
#pragma unroll
        for (int i = 0; i < ROUTE_MAX_NPL; ++i)
            if (eligible[i]) top2_merge(s1, s2, 1.0 / (1.0 + exp(-static_cast<double>(v[i]))), -1.0);
        for (int m = 1; m < lpg; m <<= 1) {
            const double b1 = __shfl_xor(s1, m, WAVE);
            const double b2 = __shfl_xor(s2, m, WAVE);
            top2_merge(s1, s2, b1, b2);
        }
        const double score = s1 + s2;
        const int my_group = lane / lpg;
        int rank = 0;
        for (int g = 0; g < n_group; ++g) {
            const double sg = __shfl(score, g * lpg, WAVE);
            if (sg > score || (sg == score && g < my_group)) ++rank;
        }
        const bool kept = my_group < n_group && rank < topk_group;
#pragma unroll
        for (int i = 0; i < ROUTE_MAX_NPL; ++i) eligible[i] = eligible[i] && kept;
    }

    uint64_t key[ROUTE_MAX_NPL];
#pragma unroll
    for (int i = 0; i < ROUTE_MAX_NPL; ++i) key[i] = eligible[i] ? route_key(v[i], lane * npl + i) : 0ull;

    int my_e = 0;
    float my_v = 0.0f, vmax = 0.0f;
    for (int r = 0; r < k; ++r) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < ROUTE_MAX_NPL; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
        const int e = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best));
        const float val = route_key_to_f32(static_cast<uint32_t>(best >> 32));
#pragma unroll
        for (int i = 0; i < ROUTE_MAX_NPL; ++i)
            if (key[i] == best) key[i] = 0ull;
        if (r == 0) vmax = val;
        if (lane == r) {
            my_e = e;
            my_v = val;
        }
    }

    if (kind == MOE355_ROUTE_SOFTMAX_TOPK) {
        const float p = lane < k ? expf(my_v - vmax) : 0.0f;
        const float sum = wave_sum_f32(p);
        *w_out = p / sum;
    } else {
        const double s = lane < k ? 1.0 / (1.0 + exp(-static_cast<double>(my_v))) : 0.0;
        double sum = s;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, WAVE);
        *w_out = static_cast<float>(s / sum * static_cast<double>(route_scale));
    }
    return my_e;
}

// Host-side check of the routing parameters (shared by every entry point that routes).
moe355_status check_route(const moe355_layer_desc* d);

}  // namespace moe355
