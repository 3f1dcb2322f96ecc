// Wavefront-level router shared by the route kernel and the fused
// route + classify kernel (included by both translation units).
//
// [Edge0, section 2 "MoE routing"]: softmax-top-k takes an exact softmax over
// the E logits, keeps the k best and renormalises; sigmoid-group scores experts
// with a sigmoid, ranks groups by the sum of their two best scores, keeps the
// best topk_group groups, picks the top k inside them and renormalises the raw
// sigmoid scores with a scale factor.
//
// Lane l owns experts [l*npl, l*npl + npl), npl = ceil(E / 64) <= 8, kept
// sorted; a selection round compares only the lanes' best entries (wavefront
// maximum of the order-preserving float bits, then wavefront minimum of the
// expert ids that hold it), so equal logits go to the lower id.  Group scores are formed in double precision from
// the float logits; expert ranking uses the float logits.
#pragma once

#include "internal.h"

namespace moe355 {

constexpr int ROUTE_MAX_NPL = 8;

__device__ __forceinline__ float route_key_to_f32(uint32_t k) {
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

// Top-2 merge of (a1 >= a2) with (b1 >= b2).
__device__ __forceinline__ void top2_merge(double& a1, double& a2, double b1, double b2) {
    const double hi = fmax(a1, b1);
    const double lo = fmax(fmin(a1, b1), fmax(a2, b2));
    a1 = hi;
    a2 = lo;
}

// Route one token with one wavefront, NPL >= npl entries per lane.  Lane j < k
// receives the j-th selected expert and its weight; the return value is that
// expert id (meaningful for lanes < k only).
template <int NPL>
__device__ __forceinline__ int route_token_n(const float* __restrict__ lg, int E, int npl, int k,
                                             int kind, int n_group, int topk_group,
                                             float route_scale, float* w_out) {
    const int lane = threadIdx.x & (WAVE - 1);
    float v[NPL];
    bool eligible[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = lane * npl + i;
        eligible[i] = i < npl && e < E;
        v[i] = eligible[i] ? lg[e] : 0.0f;
    }

    if (kind == MOE355_ROUTE_SIGMOID_GROUP) {
        const int gsize = E / n_group;
        const int lpg = gsize / npl;  // lanes per group (power of two, checked on the host)
        double s1 = -1.0, s2 = -1.0;  // sigmoid scores are > 0, so -1 is "none"
#pragma unroll
        for (int i = 0; i < NPL; ++i)
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
        for (int i = 0; i < NPL; ++i) eligible[i] = eligible[i] && kept;
    }

    // Each lane sorts its entries by (order-preserving float key descending, id
    // ascending); an ineligible entry has key 0 and id 0xFFFF, after every
    // eligible one.  A round then only looks at the lanes' heads: a DPP maximum
    // of the head keys, a DPP minimum of the ids of the heads holding it (the
    // order of value, then lower id), and the winning lane moves to its next.
    uint32_t key[NPL], id[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        key[i] = eligible[i] ? f32_order_key(v[i]) : 0u;
        id[i] = eligible[i] ? static_cast<uint32_t>(lane * npl + i) : 0xFFFFu;
    }
#pragma unroll
    for (int a = 0; a < NPL; ++a)
#pragma unroll
        for (int b = NPL - 1; b > a; --b) {
            const bool swap = key[b] > key[b - 1] || (key[b] == key[b - 1] && id[b] < id[b - 1]);
            const uint32_t k0 = key[b - 1], i0 = id[b - 1];
            key[b - 1] = swap ? key[b] : k0;
            id[b - 1] = swap ? id[b] : i0;
            key[b] = swap ? k0 : key[b];
            id[b] = swap ? i0 : id[b];
        }

    int my_e = 0;
    float my_v = 0.0f, vmax = 0.0f;
    for (int r = 0; r < k; ++r) {
        const uint32_t best = wave_max_u32(key[0]);
        const uint32_t e = wave_min_u32(key[0] == best ? id[0] : ~0u);
        if (id[0] == e) {   // the winning lane's next entry becomes its head
#pragma unroll
            for (int i = 0; i + 1 < NPL; ++i) {
                key[i] = key[i + 1];
                id[i] = id[i + 1];
            }
            key[NPL - 1] = 0u;
            id[NPL - 1] = 0xFFFFu;
        }
        const float val = route_key_to_f32(best);
        if (r == 0) vmax = val;
        if (lane == r) {
            my_e = e == 0xFFFFu ? -1 : static_cast<int>(e);
            my_v = val;
        }
    }

    if (kind == MOE355_ROUTE_SOFTMAX_TOPK) {
        const float p = lane < k ? expf(my_v - vmax) : 0.0f;
        const float sum = wave_sum_dpp_f32(p);
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

__device__ __forceinline__ int route_token(const float* __restrict__ lg, int E, int k, int kind,
                                           int n_group, int topk_group, float route_scale,
                                           float* w_out) {
    const int npl = (E + WAVE - 1) / WAVE;
    if (npl <= 1) return route_token_n<1>(lg, E, npl, k, kind, n_group, topk_group, route_scale, w_out);
    if (npl <= 2) return route_token_n<2>(lg, E, npl, k, kind, n_group, topk_group, route_scale, w_out);
    if (npl <= 4) return route_token_n<4>(lg, E, npl, k, kind, n_group, topk_group, route_scale, w_out);
    return route_token_n<ROUTE_MAX_NPL>(lg, E, npl, k, kind, n_group, topk_group, route_scale, w_out);
}

// Host-side check of the routing parameters (shared by every entry point that routes).
moe355_status check_route(const moe355_layer_desc* d);

}  // namespace moe355
