// Prefill bucketing: a stable counting sort of the T*k (token, slot) pairs by
// expert, so the grouped GEMM can run each expert once over its token bucket
// (the whole-layer prefill path of [Edge0, section 3.1 "Executor paths"] runs
// every expert of the layer over the tokens routed to it).
//
// Three small kernels: per-chunk histograms in LDS, one workgroup that turns
// them into per-chunk bases and the expert offsets, and a scatter in which one
// wavefront walks its chunk in order, 64 pairs at a time, ranking equal ids
// inside each group of 64 with ballots so the sort stays stable.
#include "internal.h"

namespace moe355 {
namespace {

constexpr int PCHUNK = 1024;

__global__ void __launch_bounds__(256) perm_count_kernel(const int32_t* __restrict__ ids, int n,
                                                         int E, int32_t* __restrict__ hist) {
    extern __shared__ int32_t h[];
    for (int e = threadIdx.x; e < E; e += blockDim.x) h[e] = 0;
    __syncthreads();
    const int beg = blockIdx.x * PCHUNK;
    for (int i = beg + threadIdx.x; i < beg + PCHUNK && i < n; i += blockDim.x) {
        const int e = ids[i];
        if (e >= 0 && e < E) atomicAdd(&h[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[static_cast<int64_t>(blockIdx.x) * E + e] = h[e];
}

// One thread per expert walks the chunks' counts twice, SB loads in flight at a
// time (the counts come from other XCDs' stores, so each batch is a trip to the
// memory side; one load at a time made this kernel a chain of nb trips).
constexpr int SB = 16;
__global__ void __launch_bounds__(1024) perm_scan_kernel(int32_t* __restrict__ hist, int nb, int E,
                                                         int n, int32_t* __restrict__ offsets) {
    __shared__ int32_t wave_tot[16];
    const int e = threadIdx.x;
    int running = 0;
    if (e < E)
        for (int b0 = 0; b0 < nb; b0 += SB) {
            int v[SB];
#pragma unroll
            for (int j = 0; j < SB; ++j) v[j] = b0 + j < nb ? hist[static_cast<int64_t>(b0 + j) * E + e] : 0;
#pragma unroll
            for (int j = 0; j < SB; ++j) running += v[j];
        }
    // exclusive scan of the per-expert totals
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
    int inc = running;
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
        int o = __shfl_up(inc, d, WAVE);
        if (lane >= d) inc += o;
    }
    if (lane == WAVE - 1) wave_tot[w] = inc;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < w; ++i) base += wave_tot[i];
    const int excl = base + inc - running;
    if (e < E) {
        offsets[e] = excl;
        int acc = excl;   // chunk b's base for expert e: excl + the counts of chunks < b
        for (int b0 = 0; b0 < nb; b0 += SB) {
            int v[SB];
#pragma unroll
            for (int j = 0; j < SB; ++j) v[j] = b0 + j < nb ? hist[static_cast<int64_t>(b0 + j) * E + e] : 0;
#pragma unroll
            for (int j = 0; j < SB; ++j)
                if (b0 + j < nb) {
                    hist[static_cast<int64_t>(b0 + j) * E + e] = acc;
                    acc += v[j];
                }
        }
    }
    if (e == 0) offsets[E] = n;
}

__global__ void __launch_bounds__(64) perm_scatter_kernel(const int32_t* __restrict__ ids, int n,
                                                          int E, const int32_t* __restrict__ hist,
                                                          int32_t* __restrict__ perm) {
    extern __shared__ int32_t cnt[];
    const int lane = threadIdx.x;
    for (int e = lane; e < E; e += WAVE) cnt[e] = hist[static_cast<int64_t>(blockIdx.x) * E + e];
    __syncthreads();
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 1;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (WAVE - lane));
    const int beg = blockIdx.x * PCHUNK;
    // the chunk's ids, all requested before the first is ranked
    constexpr int NG = PCHUNK / WAVE;
    int idv[NG];
#pragma unroll
    for (int q = 0; q < NG; ++q) {
        const int i = beg + q * WAVE + lane;
        idv[q] = i < n ? ids[i] : -1;
    }
#pragma unroll
    for (int q = 0; q < NG; ++q) {
        const int g = beg + q * WAVE;
        if (g >= n) break;
        const int i = g + lane;
        int e = idv[q];
        const bool valid = e >= 0 && e < E;
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = valid && ((e >> b) & 1);
            const uint64_t bal = __ballot(bit);
            peers &= bit ? bal : ~bal;
        }
        if (valid) {
            const int rank = __popcll(peers & below);
            const int total = __popcll(peers);
            const int pos = cnt[e] + rank;
            perm[pos] = i;
            __builtin_amdgcn_wave_barrier();
            if (rank == total - 1) cnt[e] = pos + 1;
        }
        __builtin_amdgcn_wave_barrier();
        __syncthreads();
    }
}

}  // namespace

size_t permute_ws_bytes(int E, int T, int k) {
    const int64_t n = static_cast<int64_t>(T) * k;
    const int64_t nb = (n + PCHUNK - 1) / PCHUNK;
    return static_cast<size_t>((nb > 0 ? nb : 1) * E * sizeof(int32_t));
}

moe355_status launch_permute(const int32_t* ids, int n, int E, int32_t* perm, int32_t* offsets,
                             int32_t* hist, hipStream_t stream) {
    const int nb = (n + PCHUNK - 1) / PCHUNK;
    if (nb > 0) {
        perm_count_kernel<<<nb, 256, E * sizeof(int32_t), stream>>>(ids, n, E, hist);
        moe355_status st = check_launch("permute count");
        if (st) return st;
    }
    perm_scan_kernel<<<1, 1024, 0, stream>>>(hist, nb, E, n, offsets);
    moe355_status st = check_launch("permute scan");
    if (st) return st;
    if (nb > 0) {
        perm_scatter_kernel<<<nb, 64, E * sizeof(int32_t), stream>>>(ids, n, E, hist, perm);
        return check_launch("permute scatter");
    }
    return MOE355_OK;
}

}  // namespace moe355

using namespace moe355;

extern "C" moe355_status moe355_permute(const moe355_layer_desc* d, const int32_t* topk_ids,
                                        int32_t T, int32_t* perm, int32_t* offsets, void* ws,
                                        size_t ws_bytes, hipStream_t stream) {
    moe355_status st = check_desc(d);
    if (st) return st;
    MOE355_REQUIRE(offsets && (T == 0 || (topk_ids && perm)), MOE355_EINVAL,
                   "permute: null pointer");
    MOE355_REQUIRE(T >= 0 && static_cast<int64_t>(T) * d->top_k < (1ll << 30), MOE355_EINVAL,
                   "permute: T=%d", T);
    MOE355_REQUIRE(d->n_experts <= 1024, MOE355_ENOTSUP, "permute: E=%d > 1024", d->n_experts);
    const size_t need = permute_ws_bytes(d->n_experts, T, d->top_k);
    MOE355_REQUIRE(ws && ws_bytes >= need, MOE355_ECAPACITY, "permute: workspace %zu < %zu",
                   ws_bytes, need);
    return launch_permute(topk_ids, T * d->top_k, d->n_experts, perm, offsets,
                          static_cast<int32_t*>(ws), stream);
}
