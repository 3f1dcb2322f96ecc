// The HBM expert cache's per-call bookkeeping, fill copy and elastic rebuild.
//
// [FT-zh, Core method / Method steps]: per layer call, on the device: dedup the
// routed ids, classify them against the slot table into hits and misses,
// split the misses into a fill set F (q experts) and an in-place set C, select
// K LRU victims with one scan, and batch-copy F into the first q victims.
// [FT-en, Semantic-Aware Expert Caching]: recency moves only on a router
// selection.  [FT-en, Elastic Memory Management]: one scan returns the K
// oldest slots, the miss path consumes the first q, reused slots take the
// current step as timestamp; a smaller budget evicts excess slots at a safe
// point without a restart.
//
// classify_evict is one workgroup of 1024 threads.  Every slot timestamp is
// read from HBM once into LDS; hits are stamped in LDS; the K smallest
// (ts, slot) keys among slots with ts < tick are found by an 8-bit-digit radix
// select over LDS histograms, then ranked by counting.  Owning the whole call
// in one workgroup keeps the table updates free of cross-workgroup atomics.
#include <utility>

#include "classify_dev.h"

namespace moe355 {
namespace {

constexpr int CL_THREADS = 1024;
constexpr int CL_WAVES = CL_THREADS / WAVE;

// Exclusive block scan over CL_THREADS threads (all threads must call it).
__device__ uint64_t block_excl_scan(uint64_t v, uint64_t* wave_tot, uint64_t* total) {
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
    uint64_t inc = v;
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
        uint64_t o = __shfl_up(inc, d, WAVE);
        if (lane >= d) inc += o;
    }
    if (lane == WAVE - 1) wave_tot[w] = inc;
    __syncthreads();
    uint64_t base = 0, all = 0;
    for (int i = 0; i < CL_WAVES; ++i) {
        uint64_t t = wave_tot[i];
        if (i < w) base += t;
        all += t;
    }
    *total = all;
    __syncthreads();
    return base + inc - v;
}

__device__ uint32_t block_sum_u32(uint32_t v, uint32_t* red) {
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
    if (lane == 0) red[w] = v;
    __syncthreads();
    uint32_t s = 0;
    for (int i = 0; i < CL_WAVES; ++i) s += red[i];
    __syncthreads();
    return s;
}

__device__ uint64_t block_max_u64(uint64_t v, uint64_t* red) {
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
    v = wave_max_u64(v);
    if (lane == 0) red[w] = v;
    __syncthreads();
    uint64_t s = 0;
    for (int i = 0; i < CL_WAVES; ++i) s = red[i] > s ? red[i] : s;
    __syncthreads();
    return s;
}

struct SelectScratch {
    uint32_t hist[256];
    uint32_t pick[2];  // chosen digit, remaining rank
    uint64_t red[CL_WAVES];
    uint32_t red32[CL_WAVES];
};

// Key of slot s: valid(s) ? (ts(s) << sbits | s) : none.  Returns the `rank`-th
// smallest valid key (1-based); all keys are distinct and below 2^bits.  `rank`
// must be in [1, number of valid keys].  Two barriers per 8-bit digit: wave 0
// scans the histogram, picks the digit and clears the histogram for the next.
template <typename KeyFn>
__device__ uint64_t radix_select(int n, uint32_t rank, int bits, KeyFn key_of, SelectScratch* sc) {
    for (int i = threadIdx.x; i < 256; i += CL_THREADS) sc->hist[i] = 0;
    __syncthreads();
    int shift = ((bits > 0 ? bits - 1 : 0) / 8) * 8;
    uint64_t prefix = 0, pmask = 0;
    uint32_t remaining = rank;
    for (; shift >= 0; shift -= 8) {
        for (int s = threadIdx.x; s < n; s += CL_THREADS) {
            uint64_t k;
            if (key_of(s, &k) && (k & pmask) == prefix)
                atomicAdd(&sc->hist[(k >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (threadIdx.x < WAVE) {
            const int lane = threadIdx.x;
            uint32_t c[4], local = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                c[i] = sc->hist[lane * 4 + i];
                local += c[i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) sc->hist[lane * 4 + i] = 0;
            uint32_t inc = local;
#pragma unroll
            for (int d = 1; d < WAVE; d <<= 1) {
                uint32_t o = __shfl_up(inc, d, WAVE);
                if (lane >= d) inc += o;
            }
            uint32_t before = inc - local;
            // the lane whose range crosses `remaining` records the digit
            if (before < remaining && remaining <= inc) {
                uint32_t acc = before;
                for (int i = 0; i < 4; ++i) {
                    if (acc + c[i] >= remaining) {
                        sc->pick[0] = lane * 4 + i;
                        sc->pick[1] = remaining - acc;
                        break;
                    }
                    acc += c[i];
                }
            }
        }
        __syncthreads();
        prefix |= static_cast<uint64_t>(sc->pick[0]) << shift;
        pmask |= 255ull << shift;
        remaining = sc->pick[1];
    }
    return prefix;
}

}  // namespace

namespace {

using ClassifyShared = ClassifySharedT<MAX_SLOTS, OWN_SLOTS, MAX_EXPERTS, MAX_LIST>;

template <int SPL>
__global__ void __launch_bounds__(CL_THREADS) classify_kernel(ClassifyParams cp) {
    __shared__ ClassifyShared sh;
    classify_body<SPL, CL_THREADS>(cp, sh, nullptr, nullptr);
}

}  // namespace

namespace {

// Copy 16-byte units [b, e) of src to dst by a 256-thread block: eight loads in
// flight per thread, then non-temporal stores (the copied bytes are not read
// again by this launch).
__device__ __forceinline__ void copy_units(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                           int64_t b, int64_t e) {
    typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
    constexpr int U = 8;
    for (int64_t base = b + threadIdx.x; base < e; base += 256 * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (base + 256 * u < e) v[u] = src[base + 256 * u];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (base + 256 * u < e)
                __builtin_nontemporal_store(u32x4v{v[u].x, v[u].y, v[u].z, v[u].w},
                                            reinterpret_cast<u32x4v*>(dst + base + 256 * u));
    }
}

// Copy the filled experts' bytes from the pool into their slots.
__global__ void __launch_bounds__(256)
fill_kernel(const uint8_t* __restrict__ pool, uint8_t* __restrict__ slots, int64_t S, int E,
            int layer, const int32_t* __restrict__ fill_e, const int32_t* __restrict__ fill_s,
            const int32_t* __restrict__ counts, int64_t chunk) {
    const int i = blockIdx.y;
    if (i >= counts[3]) return;
    const int64_t src_off = (static_cast<int64_t>(layer) * E + fill_e[i]) * S;
    const int64_t dst_off = static_cast<int64_t>(fill_s[i]) * S;
    const int64_t beg = static_cast<int64_t>(blockIdx.x) * chunk;
    const int64_t end = beg + chunk < S ? beg + chunk : S;
    copy_units(reinterpret_cast<const uint4*>(pool + src_off), reinterpret_cast<uint4*>(slots + dst_off),
               beg / 16, end / 16);
}

struct RebuildShared {
    int32_t newidx[MAX_SLOTS];
    uint64_t wave_tot[CL_WAVES];
    SelectScratch sc;
};

// Pick the to_n most recent occupied slots of `from` and lay out `to`'s tables.
__global__ void __launch_bounds__(CL_THREADS)
rebuild_select_kernel(const int32_t* __restrict__ f_table, const int32_t* __restrict__ f_owner,
                      const int64_t* __restrict__ f_ts, int f_n, int32_t* __restrict__ t_table,
                      int32_t* __restrict__ t_owner, int64_t* __restrict__ t_ts, int t_n,
                      int table_len) {
    __shared__ RebuildShared sh;
    const int tid = threadIdx.x;
    const int sbits = f_n > 1 ? 32 - __clz(f_n - 1) : 1;
    auto key_of = [&](int s, uint64_t* k) -> bool {
        *k = (static_cast<uint64_t>(f_ts[s]) << sbits) | static_cast<uint32_t>(s);
        return f_owner[s] >= 0;
    };
    uint32_t local = 0;
    for (int s = tid; s < f_n; s += CL_THREADS) local += f_owner[s] >= 0 ? 1u : 0u;
    const uint32_t n_occ = block_sum_u32(local, sh.sc.red32);
    // keep keys greater than the (n_occ - t_n)-th smallest occupied key
    uint64_t thr = 0;
    bool keep_all = n_occ <= static_cast<uint32_t>(t_n);
    if (!keep_all) {
        uint64_t mx = 0;
        for (int s = tid; s < f_n; s += CL_THREADS) {
            uint64_t k;
            if (key_of(s, &k)) mx = k > mx ? k : mx;
        }
        mx = block_max_u64(mx, sh.sc.red);
        const int bits = mx ? 64 - __clzll(static_cast<long long>(mx)) : 1;
        thr = radix_select(f_n, n_occ - t_n, bits, key_of, &sh.sc);
    }

    // new slot = rank of the kept slot in ascending old-slot order; each thread
    // owns a contiguous run of old slots so the scan follows slot order
    const int per = (f_n + CL_THREADS - 1) / CL_THREADS;
    const int s0 = tid * per;
    uint32_t cnt = 0;
    for (int s = s0; s < s0 + per && s < f_n; ++s) {
        uint64_t k;
        if (key_of(s, &k) && (keep_all || k > thr)) ++cnt;
    }
    uint64_t tot;
    uint64_t base = block_excl_scan(cnt, sh.wave_tot, &tot);
    for (int s = s0; s < s0 + per && s < f_n; ++s) {
        uint64_t k;
        if (key_of(s, &k) && (keep_all || k > thr)) {
            sh.newidx[s] = static_cast<int32_t>(base);
            t_owner[base] = f_owner[s];
            t_ts[base] = f_ts[s];
            ++base;
        } else {
            sh.newidx[s] = -1;
        }
    }
    for (int n = static_cast<int>(tot) + tid; n < t_n; n += CL_THREADS) {
        t_owner[n] = -1;
        t_ts[n] = 0;
    }
    __syncthreads();
    for (int g = tid; g < table_len; g += CL_THREADS) {
        const int s = f_table[g];
        t_table[g] = (s >= 0 && s < f_n) ? sh.newidx[s] : -1;
    }
}

// Copy the kept slots' bytes: new slot n takes the bytes of from's slot of owner[n].
__global__ void __launch_bounds__(256)
rebuild_copy_kernel(const int32_t* __restrict__ f_table, int table_len, int f_n,
                    const uint8_t* __restrict__ f_data, const int32_t* __restrict__ t_owner,
                    uint8_t* __restrict__ t_data, int64_t S, int64_t chunk) {
    const int n = blockIdx.y;
    const int g = t_owner[n];
    if (g < 0 || g >= table_len) return;
    const int s_old = f_table[g];
    if (s_old < 0 || s_old >= f_n) return;
    const int64_t beg = static_cast<int64_t>(blockIdx.x) * chunk;
    const int64_t end = beg + chunk < S ? beg + chunk : S;
    copy_units(reinterpret_cast<const uint4*>(f_data + static_cast<int64_t>(s_old) * S),
               reinterpret_cast<uint4*>(t_data + static_cast<int64_t>(n) * S), beg / 16, end / 16);
}

constexpr int64_t COPY_CHUNK = 64 * 1024;

}  // namespace

moe355_status check_out(const moe355_classify_out* o, bool full, int n_ids) {
    MOE355_REQUIRE(o && o->uniq && o->counts, MOE355_EINVAL, "classify_out: null list");
    MOE355_REQUIRE((o->plan == nullptr) == (o->pairs == nullptr), MOE355_EINVAL,
                   "classify_out: plan and pairs go together");
    MOE355_REQUIRE(o->pairs == nullptr || o->pair_capacity >= n_ids, MOE355_ECAPACITY,
                   "classify_out: pair capacity %d < %d routed ids", o->pair_capacity, n_ids);
    if (full)
        MOE355_REQUIRE(o->hit_expert && o->hit_slot && o->miss && o->fill_expert && o->fill_slot &&
                           o->inplace && o->victims,
                       MOE355_EINVAL, "classify_out: null list");
    MOE355_REQUIRE(o->capacity >= 0 && o->capacity <= MAX_LIST, MOE355_ECAPACITY,
                   "classify_out: capacity %d outside [0, %d]", o->capacity, MAX_LIST);
    return MOE355_OK;
}

moe355_status check_cache(const moe355_cache* c) {
    MOE355_REQUIRE(c && c->slot_table && c->slot_owner && c->slot_ts, MOE355_EINVAL,
                   "cache: null pointer");
    MOE355_REQUIRE(c->n_slots >= 1 && c->n_slots <= MAX_SLOTS, MOE355_ENOTSUP,
                   "cache: n_slots=%d outside [1, %d]", c->n_slots, MAX_SLOTS);
    MOE355_REQUIRE(c->n_experts >= 1 && c->n_experts <= MAX_EXPERTS, MOE355_ENOTSUP,
                   "cache: n_experts=%d outside [1, %d]", c->n_experts, MAX_EXPERTS);
    MOE355_REQUIRE(c->n_layers >= 1, MOE355_EINVAL, "cache: n_layers=%d", c->n_layers);
    MOE355_REQUIRE(static_cast<int64_t>(c->n_layers) * c->n_experts < (1ll << 31), MOE355_ENOTSUP,
                   "cache: table too large");
    return MOE355_OK;
}

// classify_evict with an optional route phase (route != null: ids are produced
// from route->logits) and an optional device-resident tick base.
moe355_status classify_setup(const moe355_cache* c, int32_t layer, const int64_t* tick_dev,
                             int64_t tick, const int32_t* ids, int32_t n_ids,
                             const moe355_evict_policy* p, moe355_classify_out* out,
                             const RouteArgs* route, ClassifyMode mode, ClassifyParams* cpp) {
    moe355_status st = check_cache(c);
    if (st) return st;
    st = check_out(out, true, n_ids);
    if (st) return st;
    MOE355_REQUIRE(p, MOE355_EINVAL, "classify_evict: null policy");
    MOE355_REQUIRE(layer >= 0 && layer < c->n_layers, MOE355_EINVAL, "classify_evict: layer=%d",
                   layer);
    if (!tick_dev)
        MOE355_REQUIRE(tick > 0 && tick < (1ll << 31), MOE355_ENOTSUP,
                       "classify_evict: tick=%lld outside (0, 2^31)", static_cast<long long>(tick));
    MOE355_REQUIRE(n_ids >= 0 && n_ids <= MAX_LIST && (n_ids == 0 || ids || route), MOE355_EINVAL,
                   "classify_evict: n_ids=%d", n_ids);
    MOE355_REQUIRE(p->K >= 0 && p->q_num >= 0 && p->q_den >= 1, MOE355_EINVAL,
                   "classify_evict: policy K=%d q=%d/%d", p->K, p->q_num, p->q_den);
    MOE355_REQUIRE(static_cast<int64_t>(p->q_num) * 2 * MAX_EXPERTS < (1ll << 62), MOE355_EINVAL,
                   "classify_evict: q_num too large");
    const int need_u = n_ids < c->n_experts ? n_ids : c->n_experts;
    const int need = need_u > p->K ? need_u : p->K;
    MOE355_REQUIRE(out->capacity >= need, MOE355_ECAPACITY,
                   "classify_evict: list capacity %d < %d", out->capacity, need);
    ClassifyParams& cp = *cpp;
    cp = ClassifyParams{};
    cp.mode = mode;
    cp.table = c->slot_table;
    cp.table_len = c->n_layers * c->n_experts;
    cp.owner = c->slot_owner;
    cp.slot_ts = c->slot_ts;
    cp.N = c->n_slots;
    cp.E = c->n_experts;
    cp.layer = layer;
    cp.tick_dev = tick_dev;
    cp.tick_add = tick;
    cp.ids = ids;
    cp.n_ids = n_ids;
    cp.K = p->K;
    cp.q_num = p->q_num;
    cp.q_den = p->q_den;
    if (route) {
        cp.logits = route->logits;
        cp.T = route->T;
        cp.k = route->k;
        cp.route_kind = route->kind;
        cp.n_group = route->n_group;
        cp.topk_group = route->topk_group;
        cp.route_scale = route->scale;
        cp.ids_out = route->ids_out;
        cp.w_out = route->w_out;
    }
    cp.uniq = out->uniq;
    cp.hit_e = out->hit_expert;
    cp.hit_s = out->hit_slot;
    cp.miss = out->miss;
    cp.fill_e = out->fill_expert;
    cp.fill_s = out->fill_slot;
    cp.inplace = out->inplace;
    cp.victims = out->victims;
    cp.counts = out->counts;
    cp.plan = out->plan;
    cp.pairs = out->pairs;
    return ok();
}

moe355_status classify_launch(const ClassifyParams& cp, hipStream_t stream) {
    const int N = cp.N;
    if (N <= 512) classify_kernel<8><<<1, CL_THREADS, 0, stream>>>(cp);
    else if (N <= 1024) classify_kernel<16><<<1, CL_THREADS, 0, stream>>>(cp);
    else if (N <= 2048) classify_kernel<32><<<1, CL_THREADS, 0, stream>>>(cp);
    else classify_kernel<0><<<1, CL_THREADS, 0, stream>>>(cp);
    return check_launch("classify_evict");
}

moe355_status classify_call(const moe355_cache* c, int32_t layer, const int64_t* tick_dev,
                            int64_t tick, const int32_t* ids, int32_t n_ids,
                            const moe355_evict_policy* p, moe355_classify_out* out,
                            const RouteArgs* route, ClassifyMode mode, hipStream_t stream) {
    ClassifyParams cp;
    const moe355_status st = classify_setup(c, layer, tick_dev, tick, ids, n_ids, p, out, route, mode, &cp);
    if (st) return st;
    return classify_launch(cp, stream);
}

}  // namespace moe355

using namespace moe355;

extern "C" moe355_status moe355_dedup(const int32_t* ids, int32_t n_ids, int32_t n_experts,
                                      moe355_classify_out* out, hipStream_t stream) {
    moe355_status st = check_out(out, false, n_ids);
    if (st) return st;
    MOE355_REQUIRE(n_ids >= 0 && n_ids <= MAX_LIST && (n_ids == 0 || ids), MOE355_EINVAL,
                   "dedup: n_ids=%d outside [0, %d]", n_ids, MAX_LIST);
    MOE355_REQUIRE(n_experts >= 1 && n_experts <= MAX_EXPERTS, MOE355_ENOTSUP,
                   "dedup: n_experts=%d", n_experts);
    const int need = n_ids < n_experts ? n_ids : n_experts;
    MOE355_REQUIRE(out->capacity >= need, MOE355_ECAPACITY, "dedup: capacity %d < %d",
                   out->capacity, need);
    ClassifyParams cp{};
    cp.mode = CLASSIFY_DEDUP;
    cp.E = n_experts;
    cp.ids = ids;
    cp.n_ids = n_ids;
    cp.q_den = 1;
    cp.uniq = out->uniq;
    cp.counts = out->counts;
    cp.plan = out->plan;
    cp.pairs = out->pairs;
    classify_kernel<8><<<1, CL_THREADS, 0, stream>>>(cp);
    return check_launch("dedup");
}

extern "C" moe355_status moe355_classify_evict(const moe355_cache* c, int32_t layer, int64_t tick,
                                               const int32_t* ids, int32_t n_ids,
                                               const moe355_evict_policy* p,
                                               moe355_classify_out* out, hipStream_t stream) {
    return classify_call(c, layer, nullptr, tick, ids, n_ids, p, out, nullptr, CLASSIFY_FULL,
                         stream);
}

namespace moe355 {
moe355_status fill_call(const moe355_cache* c, const uint8_t* pool, int32_t layer,
                        const moe355_classify_out* out, int32_t max_fill, hipStream_t stream) {
    moe355_status st = check_cache(c);
    if (st) return st;
    MOE355_REQUIRE(pool && c->slot_data && out && out->fill_expert && out->fill_slot && out->counts,
                   MOE355_EINVAL, "cache_fill: null pointer");
    MOE355_REQUIRE(layer >= 0 && layer < c->n_layers, MOE355_EINVAL, "cache_fill: layer=%d", layer);
    MOE355_REQUIRE(c->slot_bytes > 0 && c->slot_bytes % 16 == 0, MOE355_ENOTSUP,
                   "cache_fill: slot_bytes=%lld not a multiple of 16",
                   static_cast<long long>(c->slot_bytes));
    MOE355_REQUIRE(max_fill >= 0 && max_fill <= out->capacity && max_fill <= 65535,
                   MOE355_EINVAL, "cache_fill: max_fill=%d", max_fill);
    if (max_fill == 0) return ok();
    const int64_t chunks = (c->slot_bytes + COPY_CHUNK - 1) / COPY_CHUNK;
    dim3 grid(static_cast<unsigned>(chunks), static_cast<unsigned>(max_fill));
    fill_kernel<<<grid, 256, 0, stream>>>(pool, c->slot_data, c->slot_bytes, c->n_experts, layer,
                                          out->fill_expert, out->fill_slot, out->counts,
                                          COPY_CHUNK);
    return check_launch("cache_fill");
}
}  // namespace moe355

extern "C" moe355_status moe355_cache_fill(const moe355_cache* c, const uint8_t* pool,
                                           int32_t layer, const moe355_classify_out* out,
                                           int32_t max_fill, hipStream_t stream) {
    return fill_call(c, pool, layer, out, max_fill, stream);
}

extern "C" moe355_status moe355_cache_rebuild(const moe355_cache* from, moe355_cache* to,
                                              hipStream_t stream) {
    moe355_status st = check_cache(from);
    if (st) return st;
    st = check_cache(to);
    if (st) return st;
    MOE355_REQUIRE(from->n_layers == to->n_layers && from->n_experts == to->n_experts &&
                       from->slot_bytes == to->slot_bytes,
                   MOE355_EINVAL, "cache_rebuild: caches of different shape");
    MOE355_REQUIRE(from->slot_data && to->slot_data, MOE355_EINVAL, "cache_rebuild: null slot data");
    {   // `to` is written while `from` is read: no byte of the one may be a byte of the other
        const int64_t tl = static_cast<int64_t>(from->n_layers) * from->n_experts;
        auto span = [](const void* p, int64_t n) {
            const uintptr_t b = reinterpret_cast<uintptr_t>(p);
            return std::pair<uintptr_t, uintptr_t>(b, b + static_cast<uintptr_t>(n));
        };
        const std::pair<uintptr_t, uintptr_t> f[4] = {
            span(from->slot_table, tl * 4), span(from->slot_owner, int64_t{from->n_slots} * 4),
            span(from->slot_ts, int64_t{from->n_slots} * 8),
            span(from->slot_data, int64_t{from->n_slots} * from->slot_bytes)};
        const std::pair<uintptr_t, uintptr_t> t[4] = {
            span(to->slot_table, tl * 4), span(to->slot_owner, int64_t{to->n_slots} * 4),
            span(to->slot_ts, int64_t{to->n_slots} * 8),
            span(to->slot_data, int64_t{to->n_slots} * to->slot_bytes)};
        for (int i = 0; i < 4; ++i)
            for (int j = 0; j < 4; ++j)
                MOE355_REQUIRE(t[i].second <= f[j].first || f[j].second <= t[i].first, MOE355_EINVAL,
                               "cache_rebuild: array %d of the new cache overlaps array %d of the old",
                               i, j);
    }
    MOE355_REQUIRE(to->slot_bytes % 16 == 0 && to->n_slots <= 65535, MOE355_ENOTSUP,
                   "cache_rebuild: slot_bytes or n_slots unsupported");
    rebuild_select_kernel<<<1, CL_THREADS, 0, stream>>>(
        from->slot_table, from->slot_owner, from->slot_ts, from->n_slots, to->slot_table,
        to->slot_owner, to->slot_ts, to->n_slots, from->n_layers * from->n_experts);
    st = check_launch("cache_rebuild select");
    if (st) return st;
    const int64_t chunks = (to->slot_bytes + COPY_CHUNK - 1) / COPY_CHUNK;
    dim3 grid(static_cast<unsigned>(chunks), static_cast<unsigned>(to->n_slots));
    rebuild_copy_kernel<<<grid, 256, 0, stream>>>(
        from->slot_table, from->n_layers * from->n_experts, from->n_slots, from->slot_data,
        to->slot_owner, to->slot_data, to->slot_bytes, COPY_CHUNK);
    return check_launch("cache_rebuild copy");
}
