// Device side of the cache bookkeeping call, shared by the bookkeeping kernel
// and by the whole-layer decode launch that runs it in its first workgroup.
//
// [FT-zh, Core method / Method steps]: per layer call, on the device: dedup the
// routed ids, classify them against the slot table into hits and misses,
// split the misses into a fill set F (q experts) and an in-place set C, select
// K LRU victims with one scan.  [FT-en, Semantic-Aware Expert Caching]: recency
// moves only on a router selection.  [FT-en, Elastic Memory Management]: one
// scan returns the K oldest slots, the miss path consumes the first q, reused
// slots take the current step as timestamp.
#pragma once
#include <type_traits>

#include "route_dev.h"

namespace moe355 {

constexpr int MAX_SLOTS = 16384;
constexpr int MAX_EXPERTS = 1024;
constexpr int MAX_LIST = 1024;
constexpr int OWN_SLOTS = 4096;    // owners staged in LDS for caches up to this size
constexpr uint32_t SMALL_K = 16;   // up to this many victims: min rounds instead of radix select

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

// One-token plan record.  In the whole-layer launch a one-token call with at
// most REC_K routed experts and non-negative routing weights carries its whole
// plan in the plan flag: each of the flag's 64 copies is 16 words, written
// through to the device coherence point by one lane, each word with bit 31 set
// so that a reader can tell a complete copy from a cleared one (a word is
// written whole).  Word u, for the u-th smallest routed id (u < k): miss << 30
// | slot << 16 (14 bits) | id << 6 (10 bits) | the pair, i.e. the id's
// selection rank (6 bits); word 8 + u: that pair's routing weight.  Words of
// u >= k hold bit 31 alone.
constexpr int REC_K = 8;
constexpr uint32_t REC_BIT = 0x80000000u;
__host__ __device__ inline bool plan_record(const ClassifyParams& cp) {
    return cp.mode == CLASSIFY_FULL && cp.plan != nullptr && cp.pairs != nullptr &&
           cp.logits != nullptr && cp.T == 1 && cp.k >= 1 && cp.k <= REC_K && cp.N <= 16384 &&
           cp.E <= 1024 && (cp.route_kind == MOE355_ROUTE_SOFTMAX_TOPK || cp.route_scale > 0.0f);
}


namespace {

// The bookkeeping workgroup's LDS: up to NS slots (NO of them with owners
// staged), NE experts per layer and NL routed ids per call.
template <int NS, int NO, int NE, int NL>
struct ClassifySharedT {
    static constexpr int SLOTS = NS, OWN = NO, EXPERTS = NE, LIST = NL;
    uint32_t ts[NS];
    int32_t own[NO];
    int32_t tab[NE];    // this layer's row of the slot table
    int32_t mark[NE];
    int32_t upos[NE];   // expert -> its index u in uniq
    int32_t pcnt[NE];   // routed pairs per u
    int32_t pbeg[NE];   // first index of u's pairs
    int32_t ids[NL];       // the call's routed ids
    int32_t plocal[NL];    // a pair's place inside its expert's group
    int32_t miss[NL];
    uint64_t sel_key[NL];
    int32_t victims[NL];
    int32_t vic_owner[NL];
    int32_t uexp[NL];      // distinct expert u's id (lane-parallel classification)
    int32_t hslot[NL];     // the hits' slots
    int32_t n_hit;
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


// A flag raised after a device-scope release of this wavefront's stores, in 64
// copies 256 bytes apart (lane i stores copy i; the whole wavefront calls it),
// so that many pollers spread over many lines.
__device__ __forceinline__ void publish(uint32_t* flag) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_store(flag + 64 * (threadIdx.x & (WAVE - 1)), 1u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// One layer call by one workgroup of NT threads.  Phase A: every wavefront
// requests its entry of this layer's table row, the routing wavefronts (one per
// token) route.  Phase B: wavefront 0 does the bookkeeping with DPP scans and
// LDS histograms, with no workgroup barrier, while the other wavefronts stage
// every slot's timestamp and owner in LDS; they meet once, before the victim
// scan.  With pub_plan / pub_vict (a full call inside a launch whose other
// workgroups run the expert FFN), the plan as known after hit/miss
// classification is published first and the fills' victim slots second, each
// after a device-scope release.
// SPL = slots per lane the bookkeeping wavefront holds in registers (caches up
// to 64 * SPL slots); SPL = 0 reads them from LDS.
template <int SPL, int NT, class SH>
__device__ __forceinline__ void classify_body(const ClassifyParams& cp, SH& sh, uint32_t* pub_plan,
                                              uint32_t* pub_vict) {
    constexpr int NWV = NT / WAVE;
    static_assert(SH::EXPERTS <= NT, "one table entry per thread");
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
    const bool own_lds = N <= SH::OWN;
    const int n_ids = cp.logits ? cp.T * cp.k : cp.n_ids;

    // ---- phase A, every wavefront: this layer's table row, routing, clears ----
    // The table entry is requested before the logits, so the two loads are in
    // flight together (a wavefront's loads complete in order).
    const int32_t tab_v = (tid < E && !dedup_only) ? table[layer * E + tid] : -1;
    float w_tok0 = 0.0f;   // wavefront 0: token 0's routing weight of the lane's pick
    if (cp.logits) {
        for (int t = tid / WAVE; t < cp.T; t += NWV) {
            float w;
            const int e = route_token(cp.logits + static_cast<int64_t>(t) * E, E, cp.k,
                                      cp.route_kind, cp.n_group, cp.topk_group, cp.route_scale, &w);
            if (t == 0) w_tok0 = w;
            const int lane = tid & (WAVE - 1);
            if (lane < cp.k) {
                cp.ids_out[t * cp.k + lane] = e;
                cp.w_out[t * cp.k + lane] = w;
                sh.ids[t * cp.k + lane] = e;
            }
        }
    } else {
        for (int i = tid; i < n_ids; i += NT) sh.ids[i] = cp.ids[i];
    }
    if (tid < E) {
        sh.tab[tid] = tab_v;
        sh.mark[tid] = 0;
        sh.pcnt[tid] = 0;
    }
    const uint32_t tick = cp.tick_dev ? static_cast<uint32_t>(*cp.tick_dev + cp.tick_add)
                                      : static_cast<uint32_t>(cp.tick_add);
    // Victim keys (ts << sbits | slot): 32 bits when tick << sbits fits.  With
    // 32-bit keys, slots in registers and few victims, every wavefront picks the
    // K smallest keys of its own range of slots and wavefront 0 merges those.
    const int sbits = N > 1 ? 32 - __clz(N - 1) : 1;
    const bool narrow = (static_cast<uint64_t>(tick) << sbits) < (1ull << 32);
    const bool wave_sel = need_slots && SPL > 0 && narrow && K >= 1 &&
                          static_cast<uint32_t>(K) <= SMALL_K;
    static_assert(2 * SH::LIST >= NWV * static_cast<int>(SMALL_K), "candidate keys fit sel_key");
    uint32_t* const cand = reinterpret_cast<uint32_t*>(sh.sel_key);
    // Wavefront wv over slots [wv * 64 * SPW, (wv + 1) * 64 * SPW), SPW per
    // lane (consecutive, so the lanes read consecutive LDS words): the hits
    // among them take the current stamp, then K rounds of a wavefront minimum
    // over the keys above the previous pick; cand[wv * K + r] = pick r, or ~0
    // past the last eligible key.  An ineligible slot holds the key ~0, which
    // no round reaches (eligible keys are below tick << sbits < 2^32).
    auto wave_pick = [&](int wv, int ln) {
        constexpr int SPW = SPL > 0 ? (SPL + NWV - 1) / NWV : 1;
        const int wb = wv * (WAVE * SPW), we = wb + WAVE * SPW;
        for (int i = ln; i < sh.n_hit; i += WAVE) {
            const int hs = sh.hslot[i];
            if (hs >= wb && hs < we) sh.ts[hs] = tick;
        }
        wave_lds_sync();
        const int s0 = wb + ln * SPW;
        uint32_t kr[SPW];
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            const int sl = s0 + j;
            const uint32_t t = sl < N ? sh.ts[sl] : ~0u;
            kr[j] = (sl < N && t < tick) ? (t << sbits) | static_cast<uint32_t>(sl) : ~0u;
        }
        uint32_t from = 0, mine = ~0u;   // lane r keeps pick r
        for (int r = 0; r < K; ++r) {
            // min over kr[j] >= from of (kr[j] - from): the subtraction sends the
            // keys below `from` above every other
            uint32_t lm = ~0u;
#pragma unroll
            for (int j = 0; j < SPW; ++j) lm = min(lm, kr[j] - from);
            const uint32_t m = wave_min_u32(lm) + from;
            if (m == ~0u) break;
            if (ln == r) mine = m;
            from = m + 1;
        }
        if (ln < K) cand[wv * K + ln] = mine;
    };
    // with publication, the routing outputs must be complete before wavefront 0's release
    if (pub_plan) __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // ---- phase B: wavefront 0 classifies (below) while the others stage every
    // slot's timestamp and owner in LDS for the victim scan, in batches of U
    // requests per thread; the two meet at a barrier before the scan.
    if (tid >= WAVE) {
        if (need_slots) {
            constexpr int U = 8;
            const int n_st = NT - WAVE, st = tid - WAVE;
            for (int base = 0; base < N; base += n_st * U) {
                uint32_t t8[U];
                int32_t o8[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int sl = base + st + u * n_st;
                    if (sl < N) {
                        t8[u] = static_cast<uint32_t>(slot_ts[sl]);
                        if (own_lds) o8[u] = owner[sl];
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int sl = base + st + u * n_st;
                    if (sl < N) {
                        sh.ts[sl] = t8[u];
                        if (own_lds) sh.own[sl] = o8[u];
                    }
                }
            }
            __syncthreads();   // meet wavefront 0 (timestamps staged, hits known)
            if (wave_sel) {
                wave_pick(tid / WAVE, tid & (WAVE - 1));
                __syncthreads();
            }
        }
        return;
    }

    // ---- one wavefront from here on ------------------------------------------
    const int lane = tid;
    const bool with_plan = cp.plan != nullptr && cp.pairs != nullptr && !evict_only;
    auto slot_of = [&](int e) {
        const int sl = sh.tab[e];
        return (sl >= 0 && sl < N) ? sl : -1;  // an entry outside the cache counts as absent
    };

    // distinct experts (ascending ids), hits and misses, each expert's pairs
    uint32_t n_uniq = 0, n_hit = 0, n_miss = 0;
    const int epl = (E + WAVE - 1) / WAVE;   // general form: lane owns experts [e0, e1)
    const int e0 = lane * epl, e1 = min(E, e0 + epl);
    uint32_t bm = 0;                          // general form: the lane's first miss index
    // Lane-parallel form, for a full or evict-only call of at most 64 routed
    // ids: lane i holds id i; broadcasts of the ids give each its earlier and
    // total occurrences and the number of distinct ids below it (its u).  Lane
    // u then holds distinct expert u: id, slot, first pair, pair count and, for
    // a miss, its index among the misses.
    const bool small = n_ids <= WAVE && (mode == CLASSIFY_FULL || evict_only);
    int su_e = -1, su_slot = -1;
    uint32_t su_pbeg = 0, su_pcnt = 0, su_mi = 0;

    // One token, published at once: its k routed experts are distinct, so the
    // plan is those ids in ascending order, each with its slot and one pair (the
    // pair's place is its selection rank).  The bookkeeping below writes the
    // same values again, then the fills.
    bool published = false;
    if (pub_plan && mode == CLASSIFY_FULL && with_plan && cp.logits && cp.T == 1 && cp.k <= WAVE) {
        const int k = cp.k;
        const int ej = lane < k ? sh.ids[lane] : 0;
        if (__ballot(lane < k && (ej < 0 || ej >= E)) == 0) {
            uint32_t rank = 0;
            for (int j = 0; j < k; ++j) rank += __builtin_amdgcn_readlane(ej, j) < ej ? 1u : 0u;
            if (plan_record(cp)) {
                // the record in LDS (hist is free until the victim scan), then
                // lane l writes copy l
                if (lane < 2 * REC_K) sh.hist[lane] = REC_BIT;
                wave_lds_sync();
                if (lane < k) {
                    const int sl = slot_of(ej);
                    sh.hist[rank] = REC_BIT | (sl < 0 ? 1u << 30 : static_cast<uint32_t>(sl) << 16) |
                                    static_cast<uint32_t>(ej) << 6 | static_cast<uint32_t>(lane);
                    sh.hist[REC_K + rank] = __float_as_uint(w_tok0) | REC_BIT;
                }
                wave_lds_sync();
                uint32_t* dst = pub_plan + 64 * lane;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    st_dev16(dst + 4 * q, sh.hist[4 * q], sh.hist[4 * q + 1], sh.hist[4 * q + 2], sh.hist[4 * q + 3]);
            } else {
                if (lane < k) {
                    cp.uniq[rank] = ej;
                    cp.pairs[rank] = lane;
                    reinterpret_cast<int4*>(cp.plan)[rank] = make_int4(slot_of(ej), 0, static_cast<int>(rank), 1);
                }
                if (lane == 0) cp.counts[0] = k;
                publish(pub_plan);
            }
            published = true;
        }
    }

    if (small) {
        const int e = lane < n_ids ? sh.ids[lane] : -1;
        const bool valid = lane < n_ids && e >= 0 && e < E;   // ids out of range are ignored
        uint32_t before = 0, cnt = 0;
        for (int j = 0; j < n_ids; ++j) {
            const int o = __builtin_amdgcn_readlane(e, j);
            before += (o == e && j < lane) ? 1u : 0u;
            cnt += o == e ? 1u : 0u;
        }
        const uint64_t fm = __ballot(valid && before == 0);   // first occurrences
        n_uniq = static_cast<uint32_t>(__popcll(fm));
        uint32_t u = 0;
        for (uint64_t m = fm; m; m &= m - 1) u += __builtin_amdgcn_readlane(e, __builtin_ctzll(m)) < e ? 1u : 0u;
        if (valid && before == 0) {
            sh.uexp[u] = e;
            sh.pcnt[u] = static_cast<int32_t>(cnt);
        }
        wave_lds_sync();
        const bool has_u = static_cast<uint32_t>(lane) < n_uniq;
        su_e = has_u ? sh.uexp[lane] : -1;
        su_pcnt = has_u ? static_cast<uint32_t>(sh.pcnt[lane]) : 0u;
        su_slot = has_u ? slot_of(su_e) : -1;
        uint32_t n_pairs;
        su_pbeg = wave_excl_scan(su_pcnt, &n_pairs);
        const bool hit = has_u && su_slot >= 0, miss = has_u && su_slot < 0;
        const uint64_t hm = __ballot(hit), mm = __ballot(miss);
        n_hit = static_cast<uint32_t>(__popcll(hm));
        n_miss = static_cast<uint32_t>(__popcll(mm));
        const uint32_t hi = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(hm >> 32),
                                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(hm), 0u));
        su_mi = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mm >> 32),
                                          __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mm), 0u));
        if (has_u) {
            if (!evict_only) cp.uniq[lane] = su_e;
            sh.pbeg[lane] = static_cast<int32_t>(su_pbeg);
        }
        if (hit) {
            if (!evict_only) {
                cp.hit_e[hi] = su_e;
                cp.hit_s[hi] = su_slot;
            }
            sh.hslot[hi] = su_slot;
            slot_ts[su_slot] = tick;   // recency moves on a router selection
        }
        if (miss) {
            if (!evict_only) cp.miss[su_mi] = su_e;
            sh.miss[su_mi] = su_e;
        }
        if (lane == 0) sh.n_hit = static_cast<int32_t>(n_hit);
        wave_lds_sync();
        if (with_plan && valid) cp.pairs[sh.pbeg[u] + static_cast<int32_t>(before)] = lane;
        if (pub_plan && !published && mode == CLASSIFY_FULL && with_plan) {
            // first publication: where each distinct expert is read from (hits
            // from their slots, misses from the pool) and its pairs
            if (has_u)
                reinterpret_cast<int4*>(cp.plan)[lane] =
                    make_int4(su_slot, 0, static_cast<int>(su_pbeg), static_cast<int>(su_pcnt));
            if (lane == 0) cp.counts[0] = static_cast<int32_t>(n_uniq);
            publish(pub_plan);
        }
    } else {
        for (int i = lane; i < n_ids; i += WAVE) {
            const int e = sh.ids[i];
            if (e >= 0 && e < E) sh.mark[e] = 1;  // ids out of range are ignored
        }
        wave_lds_sync();

        uint32_t cu = 0, ch = 0, cm = 0;
        for (int e = e0; e < e1; ++e) {
            if (!sh.mark[e]) continue;
            ++cu;
            if (slot_of(e) >= 0) ++ch;
            else ++cm;
        }
        const uint32_t bu = wave_excl_scan(cu, &n_uniq);
        const uint32_t bh = wave_excl_scan(ch, &n_hit);
        bm = wave_excl_scan(cm, &n_miss);
        if (lane == 0) sh.n_hit = static_cast<int32_t>(n_hit);
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
                    sh.hslot[h++] = sl;
                    if (!plan_only) slot_ts[sl] = tick;  // recency moves on a router selection
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

        if (pub_plan && !published && mode == CLASSIFY_FULL && with_plan) {
            // first publication: where each distinct expert is read from (hits from
            // their slots, misses from the pool) and its pairs; the fills follow
            for (int e = e0; e < e1; ++e) {
                if (!sh.mark[e]) continue;
                const int u = sh.upos[e];
                reinterpret_cast<int4*>(cp.plan)[u] = make_int4(slot_of(e), 0, sh.pbeg[u], sh.pcnt[u]);
            }
            if (lane == 0) cp.counts[0] = static_cast<int32_t>(n_uniq);
            publish(pub_plan);
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
    __syncthreads();   // the other wavefronts have staged the timestamps and owners
    uint32_t n_vic = 0;
    if (wave_sel) {
        wave_pick(0, lane);
        __syncthreads();   // every wavefront's picks
        // the K smallest of the NWV * K candidates, in rank order (lane r keeps pick r)
        constexpr int CPL = (NWV * static_cast<int>(SMALL_K) + WAVE - 1) / WAVE;
        const int C = NWV * K;
        uint32_t c[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) c[j] = lane + j * WAVE < C ? cand[lane + j * WAVE] : ~0u;
        uint32_t from = 0;
        int vic = -1;
        for (int r = 0; r < K; ++r) {
            uint32_t lm = ~0u;
#pragma unroll
            for (int j = 0; j < CPL; ++j) lm = min(lm, c[j] - from);
            const uint32_t m = wave_min_u32(lm) + from;
            if (m == ~0u) break;
            if (lane == r) vic = static_cast<int>(m & ((1u << sbits) - 1));
            from = m + 1;
            ++n_vic;
        }
        if (static_cast<uint32_t>(lane) < n_vic) {
            sh.victims[lane] = vic;
            cp.victims[lane] = vic;
            if (own_lds) sh.vic_owner[lane] = sh.own[vic];
            else sh.vic_owner[lane] = owner[vic];
        }
        wave_lds_sync();
    } else {
        for (int i = lane; i < static_cast<int>(n_hit); i += WAVE)   // the hits' new stamps, over the staged ones
            sh.ts[sh.hslot[i]] = tick;
        wave_lds_sync();
        const int spl = SPL > 0 ? SPL : (N + WAVE - 1) / WAVE;
        const int s0 = lane * spl, s1 = min(N, s0 + spl);
        // Victims: the n_vic smallest (ts << sbits | slot) keys among eligible slots.
        // With 32-bit keys (tick << sbits fits) wavefront 0 holds every timestamp in
        // registers; otherwise it reads them from LDS.
        uint32_t n_elig = 0;
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
    if (with_plan && small) {
        // where the FFN reads each expert from after the call, and whether it is filled now
        if (static_cast<uint32_t>(lane) < n_uniq) {
            int final_slot = su_slot, filled = 0;
            if (su_slot < 0) {
                filled = su_mi < q_eff ? 1 : 0;
                final_slot = filled ? sh.victims[su_mi] : -1;
            }
            reinterpret_cast<int4*>(cp.plan)[lane] =
                make_int4(final_slot, filled, static_cast<int>(su_pbeg), static_cast<int>(su_pcnt));
        }
    } else if (with_plan) {
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
    if (pub_vict) publish(pub_vict);   // the fills' victim slots are in the plan
}

}  // namespace
}  // namespace moe355
