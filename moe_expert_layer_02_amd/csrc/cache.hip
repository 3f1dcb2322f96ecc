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
#include "route_dev.h"

namespace moe355 {
namespace {

constexpr int CL_THREADS = 1024;
constexpr int CL_WAVES = CL_THREADS / WAVE;
constexpr int MAX_SLOTS = 16384;
constexpr int MAX_EXPERTS = 1024;
constexpr int MAX_LIST = 1024;

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
// smallest valid key (1-based); all keys are distinct.  `rank` must be in
// [1, number of valid keys].
template <typename KeyFn>
__device__ uint64_t radix_select(int n, uint32_t rank, KeyFn key_of, SelectScratch* sc) {
    uint64_t mx = 0;
    for (int s = threadIdx.x; s < n; s += CL_THREADS) {
        uint64_t k;
        if (key_of(s, &k)) mx = k > mx ? k : mx;
    }
    mx = block_max_u64(mx, sc->red);
    const int bits = mx ? 64 - __clzll(static_cast<long long>(mx)) : 1;
    int shift = ((bits - 1) / 8) * 8;
    uint64_t prefix = 0, pmask = 0;
    uint32_t remaining = rank;
    for (; shift >= 0; shift -= 8) {
        for (int i = threadIdx.x; i < 256; i += CL_THREADS) sc->hist[i] = 0;
        __syncthreads();
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
        __syncthreads();
    }
    return prefix;
}

}  // namespace

struct ClassifyParams {
    int dedup_only;
    int32_t* table;
    int table_len;
    int32_t* owner;
    int64_t* slot_ts;
    int N, E, layer;
    const int64_t* tick_dev;   // tick = *tick_dev + tick_add when set, else tick_add
    int64_t tick_add;
    const int32_t* ids;
    int n_ids;
    int K, q_num, q_den;
    // optional routing of the call's tokens before the bookkeeping
    const float* logits;
    int T, k, route_kind, n_group, topk_group;
    float route_scale;
    int32_t* ids_out;
    float* w_out;
    int32_t *uniq, *hit_e, *hit_s, *miss, *fill_e, *fill_s, *inplace, *victims, *counts;
    int32_t *plan, *pairs;     // optional: the FFN's per-expert plan and grouped pairs
};

namespace {

struct ClassifyShared {
    uint32_t ts[MAX_SLOTS];
    int32_t mark[MAX_EXPERTS];
    int32_t upos[MAX_EXPERTS];   // expert -> its index u in uniq
    int32_t pcnt[MAX_EXPERTS];   // routed pairs per u
    int32_t pbeg[MAX_EXPERTS];   // first index of u's pairs
    int32_t miss[MAX_LIST];
    uint64_t sel_key[MAX_LIST];
    int32_t victims[MAX_LIST];
    uint64_t wave_tot[CL_WAVES];
    uint32_t n_sel;
    SelectScratch sc;
};

}  // namespace

// One layer call: optional routing of T tokens, then dedup, hit/miss, victims.
__global__ void __launch_bounds__(CL_THREADS) classify_kernel(ClassifyParams cp) {
    __shared__ ClassifyShared sh;
    __shared__ int32_t routed[MAX_LIST];
    const int tid = threadIdx.x;
    int32_t* __restrict__ table = cp.table;
    int32_t* __restrict__ owner = cp.owner;
    int64_t* __restrict__ slot_ts = cp.slot_ts;
    const int N = cp.N, E = cp.E, layer = cp.layer, K = cp.K, table_len = cp.table_len;
    const int dedup_only = cp.dedup_only;
    const uint32_t tick = cp.tick_dev ? static_cast<uint32_t>(*cp.tick_dev + cp.tick_add)
                                      : static_cast<uint32_t>(cp.tick_add);
    const int32_t* ids = cp.ids;
    const int n_ids = cp.n_ids;

    for (int e = tid; e < E; e += CL_THREADS) {
        sh.mark[e] = 0;
        sh.pcnt[e] = 0;
    }
    if (tid == 0) sh.n_sel = 0;
    if (cp.logits) {
        // route the call's tokens first: one wavefront per token
        for (int t = tid / WAVE; t < cp.T; t += CL_WAVES) {
            float w;
            const int e = route_token(cp.logits + static_cast<int64_t>(t) * E, E, cp.k,
                                      cp.route_kind, cp.n_group, cp.topk_group, cp.route_scale, &w);
            const int lane = tid & (WAVE - 1);
            if (lane < cp.k) {
                cp.ids_out[t * cp.k + lane] = e;
                cp.w_out[t * cp.k + lane] = w;
                routed[t * cp.k + lane] = e;
            }
        }
        ids = routed;
    }
    __syncthreads();
    for (int i = tid; i < n_ids; i += CL_THREADS) {
        int e = ids[i];
        if (e >= 0 && e < E) sh.mark[e] = 1;  // ids out of range are ignored
    }
    if (!dedup_only)
        for (int s = tid; s < N; s += CL_THREADS) sh.ts[s] = static_cast<uint32_t>(slot_ts[s]);
    __syncthreads();

    // E <= CL_THREADS: thread e handles expert e
    const int e = tid;
    const int m = (e < E) ? sh.mark[e] : 0;
    int slot = -1;
    if (m && !dedup_only) {
        slot = table[layer * E + e];
        if (slot >= N) slot = -1;  // a table entry outside the cache counts as absent
    }
    const uint64_t is_hit = (m && slot >= 0) ? 1 : 0;
    const uint64_t is_miss = (m && slot < 0) ? 1 : 0;
    const uint64_t packed = static_cast<uint64_t>(m) | (is_hit << 21) | (is_miss << 42);
    uint64_t tot;
    const uint64_t pos = block_excl_scan(packed, sh.wave_tot, &tot);
    const uint32_t n_uniq = static_cast<uint32_t>(tot & 0x1FFFFF);
    const uint32_t n_hit = static_cast<uint32_t>((tot >> 21) & 0x1FFFFF);
    const uint32_t n_miss = static_cast<uint32_t>((tot >> 42) & 0x1FFFFF);
    const int my_u = static_cast<int>(pos & 0x1FFFFF);
    if (m) {
        cp.uniq[my_u] = e;
        sh.upos[e] = my_u;
    }
    __syncthreads();

    // ---- the routed pairs of each distinct expert, grouped by u (n_ids <= threads) ----
    const bool with_plan = cp.plan != nullptr && cp.pairs != nullptr;
    int pair_u = -1, pair_local = 0;
    if (with_plan && tid < n_ids) {
        const int pe = ids[tid];
        if (pe >= 0 && pe < E) {
            pair_u = sh.upos[pe];
            pair_local = atomicAdd(&sh.pcnt[pair_u], 1);
        }
    }
    __syncthreads();
    {
        uint64_t ptot;
        const uint64_t pb = block_excl_scan(
            (with_plan && tid < static_cast<int>(n_uniq)) ? static_cast<uint64_t>(sh.pcnt[tid]) : 0ull,
            sh.wave_tot, &ptot);
        if (tid < static_cast<int>(n_uniq)) sh.pbeg[tid] = static_cast<int32_t>(pb);
    }
    __syncthreads();
    if (pair_u >= 0) cp.pairs[sh.pbeg[pair_u] + pair_local] = tid;

    if (dedup_only) {
        if (tid < 6) cp.counts[tid] = tid == 0 ? static_cast<int32_t>(n_uniq) : 0;
        if (with_plan && m)
            reinterpret_cast<int4*>(cp.plan)[my_u] = make_int4(-1, 0, sh.pbeg[my_u], sh.pcnt[my_u]);
        return;
    }
    if (is_hit) {
        const uint32_t p = (pos >> 21) & 0x1FFFFF;
        cp.hit_e[p] = e;
        cp.hit_s[p] = slot;
        sh.ts[slot] = tick;  // recency moves on a router selection
        slot_ts[slot] = tick;
    }
    if (is_miss) {
        const uint32_t p = (pos >> 42) & 0x1FFFFF;
        cp.miss[p] = e;
        sh.miss[p] = e;
    }
    __syncthreads();

    // ---- one scan of every slot's timestamp: the K oldest eligible slots ----
    const int sbits = N > 1 ? 32 - __clz(N - 1) : 1;
    auto key_of = [&](int s, uint64_t* k) -> bool {
        uint32_t t = sh.ts[s];
        *k = (static_cast<uint64_t>(t) << sbits) | static_cast<uint32_t>(s);
        return t < tick;
    };
    uint32_t local = 0;
    for (int s = tid; s < N; s += CL_THREADS) local += sh.ts[s] < tick ? 1u : 0u;
    const uint32_t n_elig = block_sum_u32(local, sh.sc.red32);
    const uint32_t n_vic = n_elig < static_cast<uint32_t>(K) ? n_elig : static_cast<uint32_t>(K);
    if (n_vic > 0) {
        uint64_t thr = ~0ull;
        if (n_elig > n_vic) thr = radix_select(N, n_vic, key_of, &sh.sc);
        for (int s = tid; s < N; s += CL_THREADS) {
            uint64_t k;
            if (key_of(s, &k) && k <= thr) {
                const uint32_t at = atomicAdd(&sh.n_sel, 1u);
                if (at < MAX_LIST) sh.sel_key[at] = k;
            }
        }
        __syncthreads();
        for (uint32_t i = tid; i < n_vic; i += CL_THREADS) {
            const uint64_t k = sh.sel_key[i];
            uint32_t r = 0;
            for (uint32_t j = 0; j < n_vic; ++j) r += sh.sel_key[j] < k ? 1u : 0u;
            const int s = static_cast<int>(k & ((1ull << sbits) - 1));
            sh.victims[r] = s;
            cp.victims[r] = s;
        }
        __syncthreads();
    }

    // ---- q split and slot update -------------------------------------------
    const int64_t q_raw = (2ll * cp.q_num * n_miss + cp.q_den) / (2ll * cp.q_den);
    const uint32_t q = static_cast<uint32_t>(q_raw < n_miss ? q_raw : n_miss);
    const uint32_t q_eff = q < n_vic ? q : n_vic;
    for (uint32_t i = tid; i < q_eff; i += CL_THREADS) {
        const int v = sh.victims[i];
        const int ex = sh.miss[i];
        const int old = owner[v];
        // evict; `old` is never one of this call's misses
        if (old >= 0 && old < table_len) table[old] = -1;
        table[layer * E + ex] = v;
        owner[v] = layer * E + ex;
        slot_ts[v] = tick;
        cp.fill_e[i] = ex;
        cp.fill_s[i] = v;
    }
    for (uint32_t i = q_eff + tid; i < n_miss; i += CL_THREADS) cp.inplace[i - q_eff] = sh.miss[i];
    if (with_plan && m) {
        // where the FFN reads this expert from after the call, and whether it is filled now
        const uint32_t p_miss = static_cast<uint32_t>((pos >> 42) & 0x1FFFFF);
        const bool filled = is_miss && p_miss < q_eff;
        const int final_slot = is_hit ? slot : (filled ? sh.victims[p_miss] : -1);
        reinterpret_cast<int4*>(cp.plan)[my_u] =
            make_int4(final_slot, filled ? 1 : 0, sh.pbeg[my_u], sh.pcnt[my_u]);
    }
    if (tid == 0) {
        cp.counts[0] = static_cast<int32_t>(n_uniq);
        cp.counts[1] = static_cast<int32_t>(n_hit);
        cp.counts[2] = static_cast<int32_t>(n_miss);
        cp.counts[3] = static_cast<int32_t>(q_eff);
        cp.counts[4] = static_cast<int32_t>(n_miss - q_eff);
        cp.counts[5] = static_cast<int32_t>(n_vic);
    }
}

namespace {

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
    const uint4* src = reinterpret_cast<const uint4*>(pool + src_off);
    uint4* dst = reinterpret_cast<uint4*>(slots + dst_off);
    for (int64_t o = beg / 16 + threadIdx.x; o < end / 16; o += blockDim.x) dst[o] = src[o];
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
    if (!keep_all) thr = radix_select(f_n, n_occ - t_n, key_of, &sh.sc);

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
    const uint4* src = reinterpret_cast<const uint4*>(f_data + static_cast<int64_t>(s_old) * S);
    uint4* dst = reinterpret_cast<uint4*>(t_data + static_cast<int64_t>(n) * S);
    for (int64_t o = beg / 16 + threadIdx.x; o < end / 16; o += blockDim.x) dst[o] = src[o];
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
moe355_status classify_call(const moe355_cache* c, int32_t layer, const int64_t* tick_dev,
                            int64_t tick, const int32_t* ids, int32_t n_ids,
                            const moe355_evict_policy* p, moe355_classify_out* out,
                            const RouteArgs* route, hipStream_t stream) {
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
    ClassifyParams cp{};
    cp.dedup_only = 0;
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
    classify_kernel<<<1, CL_THREADS, 0, stream>>>(cp);
    return check_launch("classify_evict");
}

namespace {
}  // namespace
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
    cp.dedup_only = 1;
    cp.E = n_experts;
    cp.ids = ids;
    cp.n_ids = n_ids;
    cp.q_den = 1;
    cp.uniq = out->uniq;
    cp.counts = out->counts;
    cp.plan = out->plan;
    cp.pairs = out->pairs;
    classify_kernel<<<1, CL_THREADS, 0, stream>>>(cp);
    return check_launch("dedup");
}

extern "C" moe355_status moe355_classify_evict(const moe355_cache* c, int32_t layer, int64_t tick,
                                               const int32_t* ids, int32_t n_ids,
                                               const moe355_evict_policy* p,
                                               moe355_classify_out* out, hipStream_t stream) {
    return classify_call(c, layer, nullptr, tick, ids, n_ids, p, out, nullptr, stream);
}

extern "C" moe355_status moe355_cache_fill(const moe355_cache* c, const uint8_t* pool,
                                           int32_t layer, const moe355_classify_out* out,
                                           int32_t max_fill, hipStream_t stream) {
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

extern "C" moe355_status moe355_cache_rebuild(const moe355_cache* from, moe355_cache* to,
                                              hipStream_t stream) {
    moe355_status st = check_cache(from);
    if (st) return st;
    st = check_cache(to);
    if (st) return st;
    MOE355_REQUIRE(from->n_layers == to->n_layers && from->n_experts == to->n_experts &&
                       from->slot_bytes == to->slot_bytes,
                   MOE355_EINVAL, "cache_rebuild: caches of different shape");
    MOE355_REQUIRE(from->slot_data && to->slot_data && from->slot_data != to->slot_data &&
                       from->slot_table != to->slot_table,
                   MOE355_EINVAL, "cache_rebuild: caches must be separate buffers");
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
