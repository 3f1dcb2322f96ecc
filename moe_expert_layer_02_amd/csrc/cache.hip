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
#include <type_traits>

#include "route_dev.h"

namespace moe355 {
namespace {

constexpr int CL_THREADS = 1024;
constexpr int CL_WAVES = CL_THREADS / WAVE;
constexpr int MAX_SLOTS = 16384;
constexpr int MAX_EXPERTS = 1024;
constexpr int MAX_LIST = 1024;
constexpr uint32_t SMALL_K = 16;   // up to this many victims: min rounds instead of radix select

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

struct ClassifyParams {
    int mode;                  // ClassifyMode (internal.h)
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

constexpr int OWN_SLOTS = 4096;   // owners staged in LDS for caches up to this size

struct ClassifyShared {
    uint32_t ts[MAX_SLOTS];
    int32_t own[OWN_SLOTS];
    int32_t tab[MAX_EXPERTS];    // this layer's row of the slot table
    int32_t mark[MAX_EXPERTS];
    int32_t upos[MAX_EXPERTS];   // expert -> its index u in uniq
    int32_t pcnt[MAX_EXPERTS];   // routed pairs per u
    int32_t pbeg[MAX_EXPERTS];   // first index of u's pairs
    int32_t ids[MAX_LIST];       // the call's routed ids
    int32_t plocal[MAX_LIST];    // a pair's place inside its expert's group
    int32_t miss[MAX_LIST];
    uint64_t sel_key[MAX_LIST];
    int32_t victims[MAX_LIST];
    int32_t vic_owner[MAX_LIST];
    uint32_t hist[256];
};

// Inclusive prefix sum over the 64 lanes (DPP row shifts and row broadcasts).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// Minimum over the 64 lanes (an inclusive min-scan by the same DPP steps; lane
// 63 ends with the minimum of all).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(~0u, v, 0x111, 0xf, 0xf, false)));
    v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(~0u, v, 0x112, 0xf, 0xf, false)));
    v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(~0u, v, 0x114, 0xf, 0xf, false)));
    v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(~0u, v, 0x118, 0xf, 0xf, false)));
    v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(~0u, v, 0x142, 0xa, 0xf, false)));
    v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(~0u, v, 0x143, 0xc, 0xf, false)));
    return __builtin_amdgcn_readlane(v, 63);
}

// Exclusive prefix sum and total over the 64 lanes.
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v, uint32_t* total) {
    const uint32_t inc = wave_incl_scan(v);
    *total = __builtin_amdgcn_readlane(inc, 63);
    return inc - v;
}

// Orders this wavefront's LDS accesses before the ones that follow: a compiler
// barrier plus a wait for outstanding LDS operations only (global stores stay
// in flight).
__device__ __forceinline__ void wave_lds_sync() {
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

}  // namespace

// One layer call.  All 16 wavefronts request the slot timestamps, owners and
// this layer's table row at once and route the call's tokens (one wavefront
// per token); then a single wavefront does the bookkeeping with DPP scans and
// LDS histograms, so no step after routing waits on a workgroup barrier.
// SPT = slots per thread held in registers while routing runs (caches up to
// SPT * CL_THREADS slots); SPT = 0 stores the timestamps before routing.
// SPL = slots per lane the bookkeeping wavefront holds in registers (caches up
// to 64 * SPL slots); SPL = 0 reads them from LDS.
template <int SPT, int SPL>
__global__ void __launch_bounds__(CL_THREADS) classify_kernel(ClassifyParams cp) {
    __shared__ ClassifyShared sh;
    const int tid = threadIdx.x;
    int32_t* __restrict__ table = cp.table;
    int32_t* __restrict__ owner = cp.owner;
    int64_t* __restrict__ slot_ts = cp.slot_ts;
    const int N = cp.N, E = cp.E, layer = cp.layer, K = cp.K, table_len = cp.table_len;
    const int mode = cp.mode;
    const bool dedup_only = mode == CLASSIFY_DEDUP;
    const bool plan_only = mode == CLASSIFY_PLAN;     // no cache state changes
    const bool evict_only = mode == CLASSIFY_EVICT;   // the plan is another call's
    const bool need_slots = mode == CLASSIFY_FULL || evict_only;
    const bool own_lds = N <= OWN_SLOTS;
    const int n_ids = cp.logits ? cp.T * cp.k : cp.n_ids;

    // ---- every wavefront: requests, routing, clears ---------------------------
    constexpr int R = SPT > 0 ? SPT : 1;
    int64_t ts_r[R];
    int32_t own_r[R];
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
        const int sl = tid + j * CL_THREADS;
        ts_r[j] = 0;
        own_r[j] = -1;
        if (need_slots && sl < N) {
            ts_r[j] = slot_ts[sl];
            if (own_lds) own_r[j] = owner[sl];
        }
    }
    if (SPT == 0 && need_slots) {
        for (int sl = tid; sl < N; sl += CL_THREADS) {
            sh.ts[sl] = static_cast<uint32_t>(slot_ts[sl]);
            if (own_lds) sh.own[sl] = owner[sl];
        }
    }
    for (int e = tid; e < E; e += CL_THREADS) {
        sh.tab[e] = dedup_only ? -1 : table[layer * E + e];
        sh.mark[e] = 0;
        sh.pcnt[e] = 0;
    }
    if (cp.logits) {
        for (int t = tid / WAVE; t < cp.T; t += CL_WAVES) {
            float w;
            const int e = route_token(cp.logits + static_cast<int64_t>(t) * E, E, cp.k,
                                      cp.route_kind, cp.n_group, cp.topk_group, cp.route_scale, &w);
            const int lane = tid & (WAVE - 1);
            if (lane < cp.k) {
                cp.ids_out[t * cp.k + lane] = e;
                cp.w_out[t * cp.k + lane] = w;
                sh.ids[t * cp.k + lane] = e;
            }
        }
    } else {
        for (int i = tid; i < n_ids; i += CL_THREADS) sh.ids[i] = cp.ids[i];
    }
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
        const int sl = tid + j * CL_THREADS;
        if (need_slots && sl < N) {
            sh.ts[sl] = static_cast<uint32_t>(ts_r[j]);
            if (own_lds) sh.own[sl] = own_r[j];
        }
    }
    const uint32_t tick = cp.tick_dev ? static_cast<uint32_t>(*cp.tick_dev + cp.tick_add)
                                      : static_cast<uint32_t>(cp.tick_add);
    __syncthreads();
    if (tid >= WAVE) return;

    // ---- one wavefront from here on ------------------------------------------
    const int lane = tid;
    const bool with_plan = cp.plan != nullptr && cp.pairs != nullptr && !evict_only;
    for (int i = lane; i < n_ids; i += WAVE) {
        const int e = sh.ids[i];
        if (e >= 0 && e < E) sh.mark[e] = 1;  // ids out of range are ignored
    }
    wave_lds_sync();

    // distinct experts, hits and misses; lane owns experts [e0, e0 + epl)
    const int epl = (E + WAVE - 1) / WAVE;
    const int e0 = lane * epl, e1 = min(E, e0 + epl);
    auto slot_of = [&](int e) {
        const int sl = sh.tab[e];
        return (sl >= 0 && sl < N) ? sl : -1;  // an entry outside the cache counts as absent
    };
    uint32_t cu = 0, ch = 0, cm = 0;
    for (int e = e0; e < e1; ++e) {
        if (!sh.mark[e]) continue;
        ++cu;
        if (slot_of(e) >= 0) ++ch;
        else ++cm;
    }
    uint32_t n_uniq, n_hit, n_miss;
    const uint32_t bu = wave_excl_scan(cu, &n_uniq);
    const uint32_t bh = wave_excl_scan(ch, &n_hit);
    const uint32_t bm = wave_excl_scan(cm, &n_miss);
    {
        uint32_t u = bu, h = bh, mi = bm;
        for (int e = e0; e < e1; ++e) {
            if (!sh.mark[e]) continue;
            if (!evict_only) cp.uniq[u] = e;
            sh.upos[e] = static_cast<int32_t>(u++);
            const int sl = slot_of(e);
            if (dedup_only) continue;
            if (sl >= 0) {
                if (!evict_only) {
                    cp.hit_e[h] = e;
                    cp.hit_s[h] = sl;
                }
                ++h;
                if (!plan_only) {
                    sh.ts[sl] = tick;  // recency moves on a router selection
                    slot_ts[sl] = tick;
                }
            } else {
                if (!evict_only) cp.miss[mi] = e;
                sh.miss[mi++] = e;
            }
        }
    }
    wave_lds_sync();

    // the routed pairs of each distinct expert, grouped by u
    if (with_plan) {
        for (int i = lane; i < n_ids; i += WAVE) {
            const int e = sh.ids[i];
            sh.plocal[i] = (e >= 0 && e < E) ? atomicAdd(&sh.pcnt[sh.upos[e]], 1) : -1;
        }
        wave_lds_sync();
        const int upl = (static_cast<int>(n_uniq) + WAVE - 1) / WAVE;
        const int u0 = lane * upl, u1 = min(static_cast<int>(n_uniq), u0 + upl);
        uint32_t c = 0, tot;
        for (int u = u0; u < u1; ++u) c += sh.pcnt[u];
        uint32_t b = wave_excl_scan(c, &tot);
        for (int u = u0; u < u1; ++u) {
            sh.pbeg[u] = static_cast<int32_t>(b);
            b += sh.pcnt[u];
        }
        wave_lds_sync();
        for (int i = lane; i < n_ids; i += WAVE) {
            const int e = sh.ids[i];
            if (e >= 0 && e < E) cp.pairs[sh.pbeg[sh.upos[e]] + sh.plocal[i]] = i;
        }
    }

    if (dedup_only) {
        if (lane < 6) cp.counts[lane] = lane == 0 ? static_cast<int32_t>(n_uniq) : 0;
        if (with_plan)
            for (int u = lane; u < static_cast<int>(n_uniq); u += WAVE)
                reinterpret_cast<int4*>(cp.plan)[u] = make_int4(-1, 0, sh.pbeg[u], sh.pcnt[u]);
        return;
    }
    if (plan_only) {
        // hits are read from their slots, misses from the pool; the cache is
        // updated later by the evict-only call
        if (with_plan) {
            for (int e = e0; e < e1; ++e) {
                if (!sh.mark[e]) continue;
                const int u = sh.upos[e];
                reinterpret_cast<int4*>(cp.plan)[u] = make_int4(slot_of(e), 0, sh.pbeg[u], sh.pcnt[u]);
            }
        }
        if (lane < 6) {
            const uint32_t c3[3] = {n_uniq, n_hit, n_miss};
            cp.counts[lane] = lane < 3 ? static_cast<int32_t>(c3[lane]) : 0;
        }
        return;
    }

    // ---- one scan of every slot's timestamp: the K oldest eligible slots -----
    wave_lds_sync();   // hit stamps are in LDS
    const int sbits = N > 1 ? 32 - __clz(N - 1) : 1;
    const int spl = SPL > 0 ? SPL : (N + WAVE - 1) / WAVE;
    const int s0 = lane * spl, s1 = min(N, s0 + spl);
    // Victims: the n_vic smallest (ts << sbits | slot) keys among eligible slots.
    // With 32-bit keys (tick << sbits fits) each lane holds its timestamps in
    // registers; otherwise it reads them from LDS.
    const bool narrow = (static_cast<uint64_t>(tick) << sbits) < (1ull << 32);
    uint32_t n_elig = 0, n_vic = 0;
    bool ranked = false;   // victims already written in rank order
    auto select = [&](auto key_zero, auto in_regs) {
        using KT = decltype(key_zero);
        constexpr bool REGS = decltype(in_regs)::value && SPL > 0;
        constexpr int RL = REGS ? SPL : 1;
        uint32_t tsr[RL];
        if constexpr (REGS) {
#pragma unroll
            for (int j = 0; j < SPL; j += 4) {
                if (s0 + j + 3 < N) {
                    const uint4 v = *reinterpret_cast<const uint4*>(&sh.ts[s0 + j]);
                    tsr[j] = v.x; tsr[j + 1] = v.y; tsr[j + 2] = v.z; tsr[j + 3] = v.w;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) tsr[j + i] = s0 + j + i < N ? sh.ts[s0 + j + i] : ~0u;
                }
            }
        }
        // calls f(slot, ts) for each of this lane's slots
        auto for_slots = [&](auto f) {
            if constexpr (REGS) {
#pragma unroll
                for (int j = 0; j < SPL; ++j) f(s0 + j, tsr[j]);
            } else {
                for (int sl = s0; sl < s1; ++sl) f(sl, sh.ts[sl]);
            }
        };
        uint32_t ce = 0;
        for_slots([&](int sl, uint32_t t) { ce += (sl < N && t < tick) ? 1u : 0u; });
        wave_excl_scan(ce, &n_elig);
        n_vic = n_elig < static_cast<uint32_t>(K) ? n_elig : static_cast<uint32_t>(K);
        if (n_vic == 0) return;
        constexpr int KB = 8 * sizeof(KT);
        auto key = [&](int sl, uint32_t t) { return (static_cast<KT>(t) << sbits) | static_cast<KT>(sl); };
        if constexpr (REGS && KB == 32) {
            if (n_vic <= SMALL_K) {
                // Few victims: n_vic rounds of a wave-wide minimum, each over the keys
                // above the previous pick; the picks come out in rank order.  An
                // ineligible slot holds the key ~0, which no round reaches (eligible
                // keys are below tick << sbits < 2^32 and n_vic <= n_elig).
                uint32_t kr[RL];
#pragma unroll
                for (int j = 0; j < RL; ++j)
                    kr[j] = (s0 + j < N && tsr[j] < tick) ? key(s0 + j, tsr[j]) : ~0u;
                uint32_t from = 0;   // smallest key still eligible for a pick
                int vic = -1;        // lane r keeps pick r
                for (uint32_t r = 0; r < n_vic; ++r) {
                    // min over kr[j] >= from of (kr[j] - from): the subtraction sends
                    // the keys below `from` to the top of the unsigned range
                    uint32_t lm = ~0u;
#pragma unroll
                    for (int j = 0; j < RL; ++j) lm = min(lm, kr[j] - from);
                    const uint32_t m = wave_min_u32(lm) + from;
                    if (static_cast<uint32_t>(lane) == r) vic = static_cast<int>(m & ((1u << sbits) - 1));
                    from = m + 1;
                }
                if (static_cast<uint32_t>(lane) < n_vic) {
                    sh.victims[lane] = vic;
                    cp.victims[lane] = vic;
                    if (own_lds) sh.vic_owner[lane] = sh.own[vic];
                    else sh.vic_owner[lane] = owner[vic];
                }
                ranked = true;
                return;
            }
        }
        KT thr = ~static_cast<KT>(0);
        if (n_elig > n_vic) {
            const uint64_t top = static_cast<uint64_t>(tick) << sbits;
            const int bits = 64 - __clzll(static_cast<long long>(top));
            KT prefix = 0, pmask = 0;
            uint32_t remaining = n_vic;
            for (int shift = ((bits - 1) / 8) * 8; shift >= 0; shift -= 8) {
#pragma unroll
                for (int i = 0; i < 4; ++i) sh.hist[lane * 4 + i] = 0;
                wave_lds_sync();
                for_slots([&](int sl, uint32_t t) {
                    const KT k = key(sl, t);
                    if (sl < N && t < tick && (k & pmask) == prefix)
                        atomicAdd(&sh.hist[(k >> shift) & 255u], 1u);
                });
                wave_lds_sync();
                uint32_t c4[4], local = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    c4[i] = sh.hist[lane * 4 + i];
                    local += c4[i];
                }
                uint32_t tot;
                const uint32_t before = wave_excl_scan(local, &tot);
                // the lane whose range of the histogram crosses `remaining`
                const bool mine = before < remaining && remaining <= before + local;
                uint32_t digit = 0, rem = 0;
                if (mine) {
                    uint32_t acc = before;
                    for (int i = 0; i < 4; ++i) {
                        if (acc + c4[i] >= remaining) {
                            digit = lane * 4 + i;
                            rem = remaining - acc;
                            break;
                        }
                        acc += c4[i];
                    }
                }
                const int src = __builtin_ctzll(__ballot(mine));
                digit = __builtin_amdgcn_readlane(digit, src);
                rem = __builtin_amdgcn_readlane(rem, src);
                prefix |= static_cast<KT>(digit) << shift;
                pmask |= static_cast<KT>(255) << shift;
                remaining = rem;
            }
            thr = prefix;
        }
        static_assert(KB == 32 || KB == 64, "key width");
        // collect the selected keys in slot order, then rank them by key
        uint32_t cs = 0;
        for_slots([&](int sl, uint32_t t) { cs += (sl < N && t < tick && key(sl, t) <= thr) ? 1u : 0u; });
        uint32_t n_sel;
        uint32_t at = wave_excl_scan(cs, &n_sel);
        for_slots([&](int sl, uint32_t t) {
            if (sl < N && t < tick && key(sl, t) <= thr) sh.sel_key[at++] = static_cast<uint64_t>(key(sl, t));
        });
    };
    if (narrow)
        select(uint32_t{0}, std::true_type{});
    else
        select(uint64_t{0}, std::false_type{});
    if (n_vic > 0 && ranked) wave_lds_sync();   // lane 0 wrote the victims
    if (n_vic > 0 && !ranked) {
        wave_lds_sync();
        for (uint32_t i = lane; i < n_vic; i += WAVE) {
            const uint64_t k = sh.sel_key[i];
            uint32_t r = 0;
            for (uint32_t j = 0; j < n_vic; ++j) r += sh.sel_key[j] < k ? 1u : 0u;
            const int sl = static_cast<int>(k & ((1ull << sbits) - 1));
            sh.victims[r] = sl;
            cp.victims[r] = sl;
            // owners looked up here, off the collection loop, from LDS or from
            // memory by a uniform branch (a generic load would wait for every
            // store in flight)
            if (own_lds) sh.vic_owner[r] = sh.own[sl];
            else sh.vic_owner[r] = owner[sl];
        }
        wave_lds_sync();
    }

    // ---- q split and slot update -------------------------------------------
    const int64_t q_raw = (2ll * cp.q_num * n_miss + cp.q_den) / (2ll * cp.q_den);
    const uint32_t q = static_cast<uint32_t>(q_raw < n_miss ? q_raw : n_miss);
    const uint32_t q_eff = q < n_vic ? q : n_vic;
    for (uint32_t i = lane; i < q_eff; i += WAVE) {
        const int v = sh.victims[i];
        const int ex = sh.miss[i];
        const int old = sh.vic_owner[i];
        // evict; `old` is never one of this call's misses
        if (old >= 0 && old < table_len) table[old] = -1;
        table[layer * E + ex] = v;
        owner[v] = layer * E + ex;
        slot_ts[v] = tick;
        cp.fill_e[i] = ex;
        cp.fill_s[i] = v;
    }
    for (uint32_t i = q_eff + lane; i < n_miss; i += WAVE) cp.inplace[i - q_eff] = sh.miss[i];
    if (with_plan) {
        // where the FFN reads each expert from after the call, and whether it is filled now
        uint32_t mi = bm;
        for (int e = e0; e < e1; ++e) {
            if (!sh.mark[e]) continue;
            const int u = sh.upos[e];
            const int sl = slot_of(e);
            int final_slot = sl, filled = 0;
            if (sl < 0) {
                filled = mi < q_eff ? 1 : 0;
                final_slot = filled ? sh.victims[mi] : -1;
                ++mi;
            }
            reinterpret_cast<int4*>(cp.plan)[u] = make_int4(final_slot, filled, sh.pbeg[u], sh.pcnt[u]);
        }
    }
    if (lane == 0) {
        if (!evict_only) {
            cp.counts[0] = static_cast<int32_t>(n_uniq);
            cp.counts[1] = static_cast<int32_t>(n_hit);
            cp.counts[2] = static_cast<int32_t>(n_miss);
        }
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
                            const RouteArgs* route, ClassifyMode mode, hipStream_t stream) {
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
    const int N = cp.N;
    if (N <= 512) classify_kernel<1, 8><<<1, CL_THREADS, 0, stream>>>(cp);
    else if (N <= 1024) classify_kernel<1, 16><<<1, CL_THREADS, 0, stream>>>(cp);
    else if (N <= 2048) classify_kernel<2, 32><<<1, CL_THREADS, 0, stream>>>(cp);
    else if (N <= 4096) classify_kernel<4, 0><<<1, CL_THREADS, 0, stream>>>(cp);
    else if (N <= 8192) classify_kernel<8, 0><<<1, CL_THREADS, 0, stream>>>(cp);
    else classify_kernel<0, 0><<<1, CL_THREADS, 0, stream>>>(cp);
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
    cp.mode = CLASSIFY_DEDUP;
    cp.E = n_experts;
    cp.ids = ids;
    cp.n_ids = n_ids;
    cp.q_den = 1;
    cp.uniq = out->uniq;
    cp.counts = out->counts;
    cp.plan = out->plan;
    cp.pairs = out->pairs;
    classify_kernel<1, 8><<<1, CL_THREADS, 0, stream>>>(cp);
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
