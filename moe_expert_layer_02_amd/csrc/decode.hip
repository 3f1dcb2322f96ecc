// Decode expert FFN: streams each distinct expert's packed weights from HBM
// once, dequantises them in registers, and runs the products on MFMA so that
// one pass over an expert serves up to 16 of its routed tokens at the same cost.
//
// [Edge0, section 3.1 "Math contract"]: y = down(silu(gate(x)) * up(x)) per
// routed expert over its quantised weights.  [FT-zh, Core method / Method
// steps]: the GPU computes G = H u F from cache slots while the in-place set is
// read from the pool, the partial sums merge exactly, and the misses chosen for
// filling are batch-copied into their victim slots.
//
// Products.  v_mfma_f32_16x16x32 with the weights as the A operand (16 rows x
// 32 inputs) and the routed tokens as B (32 inputs x 16 tokens).  A wavefront
// load of 16 rows x 64 bytes (one "slab" of 128 inputs) gives every lane one
// 16-byte chunk, which feeds four MFMA steps.
//   int4 g64 (f16 MFMA): the A value is s * (q - 8), exact in f16 for any bf16
//     scale (|q - 8| <= 8 keeps the product within 11 significant bits); the
//     bias term sum_g (b_g + 8 s_g) * sum_{k in g} x_k goes through one more
//     MFMA per slab on hi/lo f16 splits of both factors.  x is converted to
//     f16 (exact for bf16 values in f16's range).
//   MXFP4 (bf16 MFMA): the gfx950 scaled fp4 -> bf16 conversion applies the
//     e8m0 block scale and is exact; x is bf16 already.
// h = silu(g) * u crosses into the down projection as a hi/lo pair of 16-bit
// values (f16 for int4, bf16 for MXFP4), and the down pass runs both halves.
//
// Two launches:
//   gate/up: a block item is (distinct expert, tile of I rows); the block's
//     four wavefronts split H into KW parts (and the rows into 4/KW groups),
//     reduce their partial sums through LDS and write h.  It also zeroes the
//     layer output.
//   down + combine: a wavefront item is (distinct expert, tile of H rows) over
//     all of I (with many distinct experts, units of 64 rows dealt to the
//     blocks in balanced ranges, h staged in LDS); each row's result meets the
//     routing weight and is added into the fp32 layer output with an atomic
//     (k additions per element).
// Each block stages the call's plan (for each distinct expert: where its bytes
// live, whether this call fills a cache slot with it, its routed pairs) in LDS
// first, so every weight load is independent of the others, and each
// wavefront keeps the loads of the next two or three slabs in flight while it
// computes one.  With
// fill-through on, an expert that this call fills into a cache slot is read
// from the pool and the lanes that read its bytes also write them to the slot.
#include "internal.h"
#include "classify_dev.h"

namespace moe355 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int SLAB = 128;   // inputs per wavefront load (16 rows x 64 bytes)
constexpr int TOK = 16;     // tokens per MFMA pass

struct DecodeParams {
    const uint16_t* x;       // [T][H] bf16
    const float* w;          // [T*k] routing weights
    const int32_t* uniq;
    const int32_t* counts;
    const uint8_t* slots;
    const uint8_t* pool;
    const int32_t* plan;     // [n_plan][4]: slot or -1, filled now, first pair, pair count
    const int32_t* pairs;    // routed pairs grouped by expert
    int n_plan;              // plan rows loaded (>= number of distinct experts)
    int has_cache;
    int fill_through;
    int64_t S;
    int E, layer, T, k, H, I;
    int64_t q_off[3], s_off[3], b_off[3];
    uint16_t* h_hi;          // [T*k][I] high half of h (f16 for int4, bf16 for MXFP4)
    uint16_t* h_lo;          // [T*k][I] remainder h - h_hi
    float* out;              // [T][H]
    uint32_t* err;           // the workspace's sticky error word
};

// Device-memory (address space 1) byte pointers: loads and stores through them
// compile to global instructions, which, unlike generic ones, do not count
// against the LDS wait counter.
typedef __attribute__((address_space(1))) const uint8_t* gbytes;
typedef __attribute__((address_space(1))) uint8_t* gbytes_w;

struct ExpertRef {
    gbytes src;
    gbytes_w dst;  // fill-through destination slot, or null
};

// The per-call plan, staged in LDS by every block before any weight load.
constexpr int MAX_PLAN = 256;
struct PlanLds {
    int4 plan[MAX_PLAN];
    int32_t uniq[MAX_PLAN];
    int32_t pairs[MAX_PLAN];
    int32_t tok[MAX_PLAN];   // token of pairs[i] (pairs[i] / k)
    float w[MAX_PLAN];       // routing weight of each pair
    int32_t n_uniq;
    int32_t fills_known;     // whole-layer launch: the staged plan already names the fills
    uint32_t rec[2 * REC_K]; // whole-layer launch: the one-token plan record
};

// A wavefront-uniform device pointer moved into scalar registers, so that loads
// from it take a 32-bit per-lane offset instead of 64-bit per-lane arithmetic.
__device__ __forceinline__ uint64_t uniform_addr(const void* q) {
    const uint64_t v = reinterpret_cast<uint64_t>(q);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Where distinct expert u's bytes are read from (and written to, with fill-through).
// u is wavefront-uniform, so are both pointers.
__device__ __forceinline__ ExpertRef expert_ref(const DecodeParams& p, const PlanLds& pl, int u) {
    const int4 row = pl.plan[u];
    ExpertRef r;
    const uint8_t* src = p.pool + (static_cast<int64_t>(p.layer) * p.E + pl.uniq[u]) * p.S;
    const uint8_t* dst = nullptr;
    if (p.has_cache && row.x >= 0) {
        const uint8_t* slot = p.slots + static_cast<int64_t>(row.x) * p.S;
        if (p.fill_through && row.y)
            dst = slot;          // filled by this call: read the pool, write the slot
        else
            src = slot;
    }
    r.src = reinterpret_cast<gbytes>(uniform_addr(src));
    r.dst = reinterpret_cast<gbytes_w>(uniform_addr(dst));
    return r;
}

__device__ __forceinline__ void stage_plan(const DecodeParams& p, PlanLds& pl) {
    if (threadIdx.x < p.n_plan) {
        pl.plan[threadIdx.x] = reinterpret_cast<const int4*>(p.plan)[threadIdx.x];
        pl.uniq[threadIdx.x] = p.uniq[threadIdx.x];
    }
    if (threadIdx.x < p.T * p.k) {
        pl.pairs[threadIdx.x] = p.pairs[threadIdx.x];
        pl.tok[threadIdx.x] = p.pairs[threadIdx.x] / p.k;
        pl.w[threadIdx.x] = p.w[threadIdx.x];
    }
    if (threadIdx.x == 0) pl.n_uniq = p.counts[0];
    __syncthreads();
}

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint32_t ldg4(const void* p) { return *reinterpret_cast<const uint32_t*>(p); }
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldg16(gbytes p) {
    const u32x4_t v = *reinterpret_cast<__attribute__((address_space(1))) const u32x4_t*>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ldg4(gbytes p) {
    return *reinterpret_cast<__attribute__((address_space(1))) const uint32_t*>(p);
}
// Fill-through stores (an expert's bytes into its cache slot, not read again in
// this call): non-temporal, so they stream out instead of settling in the L2
// (measured: the DS-like decode step 3.7 % faster than with plain stores).
__device__ __forceinline__ void stg16(gbytes_w p, const uint4& v) {
    __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w},
                                reinterpret_cast<__attribute__((address_space(1))) u32x4_t*>(p));
}
__device__ __forceinline__ void stg4(gbytes_w p, uint32_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<__attribute__((address_space(1))) uint32_t*>(p));
}
__device__ __forceinline__ uint32_t as_u32(half2_t v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ uint32_t as_u32(bf16x2_t v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

template <int FMT>
__device__ __forceinline__ f32x4 mma(uint4 a, uint4 b, f32x4 c) {
    if (FMT == MOE355_W_INT4_G64)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                      __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
    return e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
}

// f16 pair from two fp32 values that are exact in f16.
__device__ __forceinline__ uint32_t pk_f16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// int4: f16(s * (q - 8)) for the 8 codes of one dword, in the order
// (0,4,1,5,2,6,3,7) of their place in the dword.  |q - 8| <= 8 keeps every
// product of a bf16 scale within f16's 11 significant bits, so each value is
// exact; the offset moves into the bias (b + 8 s).
__device__ __forceinline__ uint4 a_int4(uint32_t d, half2_t s2) {
    const half2_t off = {static_cast<_Float16>(-1032.0f), static_cast<_Float16>(-1032.0f)};
    uint32_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const half2_t q = as_h2(((d >> (4 * i)) & 0x000F000Fu) | 0x64006400u);  // 1024 + q
        v[i] = as_u32((q + off) * s2);
    }
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// MXFP4: the 8 codes of one dword, scaled by 2^(e-127), exact in bf16, natural order.
__device__ __forceinline__ uint4 a_fp4(uint32_t d, float scale) {
    return make_uint4(as_u32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 0)),
                      as_u32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 1)),
                      as_u32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 2)),
                      as_u32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 3)));
}

// 8 bf16 activations (natural order) as f16 in the int4 A order, plus their sum.
__device__ __forceinline__ uint4 b_x_f16(uint4 v, float* sum) {
    const half2_t one = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
    const uint32_t p0 = pk_f16(__uint_as_float(v.x << 16), __uint_as_float(v.z << 16));
    const uint32_t p1 = pk_f16(__uint_as_float(v.x & 0xFFFF0000u), __uint_as_float(v.z & 0xFFFF0000u));
    const uint32_t p2 = pk_f16(__uint_as_float(v.y << 16), __uint_as_float(v.w << 16));
    const uint32_t p3 = pk_f16(__uint_as_float(v.y & 0xFFFF0000u), __uint_as_float(v.w & 0xFFFF0000u));
    float s = *sum;
    s = __builtin_amdgcn_fdot2(as_h2(p0), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(p1), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(p2), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(p3), one, s, false);
    *sum = s;
    return make_uint4(p0, p1, p2, p3);
}

__device__ __forceinline__ float sum_f16x8(uint4 v, float s) {
    const half2_t one = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
    s = __builtin_amdgcn_fdot2(as_h2(v.x), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(v.y), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(v.z), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(v.w), one, s, false);
    return s;
}

// The slab's two group sums of a lane's 32 values (chunks 0,1 -> first group,
// chunks 2,3 -> second), as the bias MFMA's B operand: lanes of chunk 0 hold
// [hi0, hi1, lo0, lo1, hi0, hi1, 0, 0]; every other lane holds zeros.
__device__ __forceinline__ uint4 bias_b_operand(float part, int gq) {
    float v = part + __shfl_xor(part, 16, WAVE);
    const float o = __shfl_xor(v, 32, WAVE);
    const float g0 = gq < 2 ? v : o, g1 = gq < 2 ? o : v;
    const _Float16 h0 = static_cast<_Float16>(g0), h1 = static_cast<_Float16>(g1);
    const _Float16 l0 = static_cast<_Float16>(g0 - static_cast<float>(h0));
    const _Float16 l1 = static_cast<_Float16>(g1 - static_cast<float>(h1));
    if (gq != 0) return make_uint4(0u, 0u, 0u, 0u);
    const half2_t hi = {h0, h1}, lo = {l0, l1};
    return make_uint4(as_u32(hi), as_u32(lo), as_u32(hi), 0u);
}

// The bias MFMA's A operand for one row and the slab's two groups: b' = b + 8 s
// (exact in fp32) as an f16 hi/lo pair, laid out [h0, h1, h0, h1, l0, l1, 0, 0]
// against the B operand above (the lo x lo term is below f16's resolution).
__device__ __forceinline__ uint4 bias_a_operand(uint32_t bd, uint32_t sd, int gq) {
    if (gq != 0) return make_uint4(0u, 0u, 0u, 0u);
    const float b0 = __uint_as_float(bd << 16) + 8.0f * __uint_as_float(sd << 16);
    const float b1 = __uint_as_float(bd & 0xFFFF0000u) + 8.0f * __uint_as_float(sd & 0xFFFF0000u);
    const _Float16 h0 = static_cast<_Float16>(b0), h1 = static_cast<_Float16>(b1);
    const _Float16 l0 = static_cast<_Float16>(b0 - static_cast<float>(h0));
    const _Float16 l1 = static_cast<_Float16>(b1 - static_cast<float>(h1));
    const half2_t hi = {h0, h1}, lo = {l0, l1};
    return make_uint4(as_u32(hi), as_u32(hi), as_u32(lo), 0u);
}

// int4 scale of this lane's chunk as an f16 pair (s, s).
__device__ __forceinline__ half2_t int4_scale(uint32_t sd, int gq) {
    const float s = __uint_as_float(gq < 2 ? (sd << 16) : (sd & 0xFFFF0000u));
    const _Float16 sh = static_cast<_Float16>(s);
    return half2_t{sh, sh};
}

// silu(z) = z / (1 + e^-z), with the hardware reciprocal (about 1 ulp) in place
// of an IEEE division
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Loads of one slab for one matrix and RT row tiles: codes, scale dword, bias dword.
template <int RT>
struct WSlab {
    uint4 q[RT];
    uint32_t sc[RT];
    uint32_t bi[RT];
};

// Byte offsets, within a matrix's regions, of lane (ln, gq)'s part of the slab
// of rows r0 .. r0+15 (r0 a multiple of 16) at input kb (a multiple of 128): in
// the device layout that slab is one block, its codes one contiguous 1 KB (the
// lane's chunk gq of row ln at (16 gq + ln) * 16) and its scale words 64
// contiguous bytes (row ln's at 4 ln).  32-bit: a blob is far below 4 GiB.
struct SlabOff {
    uint32_t q, s;
};
__device__ __forceinline__ SlabOff slab_off(int r0, int kdim, int kb, int ln, int gq) {
    const uint32_t blk = static_cast<uint32_t>(r0 / 16) * static_cast<uint32_t>(kdim / 128) +
                         static_cast<uint32_t>(kb / 128);
    SlabOff o;
    o.q = blk * 1024u + static_cast<uint32_t>(16 * gq + ln) * 16u;
    o.s = blk * 64u + static_cast<uint32_t>(ln) * 4u;
    return o;
}

template <int FMT, int RT>
__device__ __forceinline__ void load_wslab(const DecodeParams& p, gbytes src, int m,
                                           int row0, int kdim, int kb, int ln, int gq,
                                           WSlab<RT>& w) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const SlabOff o = slab_off(row0 + 16 * t, kdim, kb, ln, gq);
        w.q[t] = ldg16(src + (static_cast<uint32_t>(p.q_off[m]) + o.q));
        w.sc[t] = ldg4(src + (static_cast<uint32_t>(p.s_off[m]) + o.s));
        // every lane loads (a broadcast within the row); only chunk-0 lanes use it
        w.bi[t] = FMT == MOE355_W_INT4_G64 ? ldg4(src + (static_cast<uint32_t>(p.b_off[m]) + o.s)) : 0u;
    }
}

// Fill-through: write a slab's bytes (codes by every lane, scale words once per row).
template <int FMT, int RT>
__device__ __forceinline__ void store_wslab(const DecodeParams& p, gbytes_w dst, int m, int row0,
                                            int kdim, int kb, int ln, int gq, const WSlab<RT>& w) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const SlabOff o = slab_off(row0 + 16 * t, kdim, kb, ln, gq);
        stg16(dst + (static_cast<uint32_t>(p.q_off[m]) + o.q), w.q[t]);
        if (gq == 0) {
            stg4(dst + (static_cast<uint32_t>(p.s_off[m]) + o.s), w.sc[t]);
            if (FMT == MOE355_W_INT4_G64) stg4(dst + (static_cast<uint32_t>(p.b_off[m]) + o.s), w.bi[t]);
        }
    }
}

// acc[t] += W_slab(row tile t) . B over the slab's four MFMA steps (B given per step).
template <int FMT, int RT>
__device__ __forceinline__ void mma_slab(const WSlab<RT>& w, const uint4 b[4], int gq,
                                         f32x4 acc[RT]) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const uint32_t d4[4] = {w.q[t].x, w.q[t].y, w.q[t].z, w.q[t].w};
        if (FMT == MOE355_W_INT4_G64) {
            const half2_t s2 = int4_scale(w.sc[t], gq);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[t] = mma<FMT>(a_int4(d4[j], s2), b[j], acc[t]);
        } else {
            const float scale = e8m0_to_f32((w.sc[t] >> (8 * gq)) & 0xFFu);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[t] = mma<FMT>(a_fp4(d4[j], scale), b[j], acc[t]);
        }
    }
}

// acc[t] += W_slab(row tile t) . (Bh + Bl): the hi and lo halves of the B
// operand against weights dequantised once.
template <int FMT, int RT>
__device__ __forceinline__ void mma_slab2(const WSlab<RT>& w, const uint4 bh[4], const uint4 bl[4],
                                          int gq, f32x4 acc[RT]) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const uint32_t d4[4] = {w.q[t].x, w.q[t].y, w.q[t].z, w.q[t].w};
        if (FMT == MOE355_W_INT4_G64) {
            const half2_t s2 = int4_scale(w.sc[t], gq);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 a = a_int4(d4[j], s2);
                acc[t] = mma<FMT>(a, bh[j], acc[t]);
                acc[t] = mma<FMT>(a, bl[j], acc[t]);
            }
        } else {
            const float scale = e8m0_to_f32((w.sc[t] >> (8 * gq)) & 0xFFu);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 a = a_fp4(d4[j], scale);
                acc[t] = mma<FMT>(a, bh[j], acc[t]);
                acc[t] = mma<FMT>(a, bl[j], acc[t]);
            }
        }
    }
}

// Synchronisation words, 256 bytes apart (so that no two share a cache line),
// in the first SYNC_BYTES of the decode workspace; zero before a call and left
// zero by it.  Word w sits at byte 256 w:
//   0..7     gate/up blocks of group g = block % 8 done
//   8        groups whose gate/up blocks are all done
//   9..16    blocks of group g = block % 8 exited
//   17       groups whose blocks have all exited; the last block to exit clears
//            every word
//   18       error word, sticky: bit 0 = a bounded wait gave up, bit 1 = an
//            int4 activation or h value outside f16's finite range
//   32..95   flag "all gate/up blocks done", one copy per line
//   96..159  whole-layer launch: flag "plan published", one copy per line (a
//            one-token call writes the whole plan as a 16-word record in each
//            copy, see plan_record)
//   160..223 whole-layer launch: flag "fills' victim slots published"
// Counting in groups keeps each counter to about 1/8 of the blocks, and a flag
// is raised in 64 copies (one store by each lane of a wavefront) of which a
// block polls copy block % 64: requests to one address are served one after
// another at the memory side, so 256 atomic additions on one counter cost
// about as much as the whole gate/up pass, and a few hundred blocks polling
// one word slow down every other access that falls on that channel.
//
// h crosses between blocks without whole-cache maintenance: the gate/up blocks
// store it with device-scope (write-through) stores and wait for their
// completion before counting themselves done; the down blocks read it with
// device-scope loads after seeing the flag.  (A release or acquire fence at
// device scope would write back or invalidate the XCD's whole L2, once per
// block.)
constexpr uint32_t SPIN_LIMIT = 1u << 18;   // polls of >= 128 cycles: tens of ms at most
constexpr int SYNC_BYTES = 65536;
__device__ __forceinline__ uint32_t* sync_word(uint32_t* sync, int w) { return sync + 64 * w; }
constexpr int SW_DONE = 0, SW_DONE_TOP = 8, SW_EXIT = 9, SW_EXIT_TOP = 17, SW_ERR = 18;
constexpr int FL_DONE = 32, FL_PLAN = 96, FL_VICT = 160;   // 64 copies each

__device__ __forceinline__ uint32_t atomic_add_dev(uint32_t* a, uint32_t v) {
    return __hip_atomic_fetch_add(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev(uint32_t* a, uint32_t v) {
    __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// blocks b < n with b % 8 == g
__device__ __forceinline__ uint32_t group_size(uint32_t n, uint32_t g) { return g < n ? (n - g + 7) / 8 : 0; }

// Gate/up block `a` (of n_gu) counts itself done once its h stores are complete;
// the block that completes the count raises the flag.
__device__ __forceinline__ void signal_done(uint32_t* sync, uint32_t n_gu, uint32_t a) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wavefront's h stores are complete
    __syncthreads();
    if (threadIdx.x < WAVE) {
        uint32_t last = 0;
        if (threadIdx.x == 0) {
            const uint32_t g = a & 7;
            if (atomic_add_dev(sync_word(sync, SW_DONE + g), 1u) == group_size(n_gu, g) - 1)
                last = atomic_add_dev(sync_word(sync, SW_DONE_TOP), 1u) == (n_gu < 8 ? n_gu : 8) - 1;
        }
        if (__shfl(last, 0, WAVE)) store_dev(sync_word(sync, FL_DONE + threadIdx.x), 1u);
    }
}

// Until copy `b % 64` of flag f is up (bounded; thread 0 polls, the block then meets).
__device__ __forceinline__ void wait_flag(uint32_t* sync, int f, uint32_t b, uint32_t* err) {
    if (threadIdx.x == 0) {
        const uint32_t* word = sync_word(sync, f + static_cast<int>(b & 63));
        uint32_t n = 0;
        while (__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
            __builtin_amdgcn_s_sleep(2);
            if (++n == SPIN_LIMIT) {
                __hip_atomic_fetch_or(err, ERR_WAIT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    __syncthreads();
}

// Whole-layer launch: until the plan flag (copy b % 64) is up, also noting
// whether the victims flag already was (then the plan about to be staged is
// final and names every fill).
__device__ __forceinline__ void wait_plan(uint32_t* sync, uint32_t b, PlanLds& pl, uint32_t* err) {
    if (threadIdx.x == 0) {
        const uint32_t* pw = sync_word(sync, FL_PLAN + static_cast<int>(b & 63));
        const uint32_t* vw = sync_word(sync, FL_VICT + static_cast<int>(b & 63));
        uint32_t n = 0, v = 0;
        while (true) {
            v = __hip_atomic_load(vw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (__hip_atomic_load(pw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) break;
            __builtin_amdgcn_s_sleep(2);
            if (++n == SPIN_LIMIT) {
                __hip_atomic_fetch_or(err, ERR_WAIT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
        pl.fills_known = v != 0u;
    }
    __syncthreads();
}

// The exit count in three steps.  exit_begin, once every thread of the block is
// past its last wait: thread 0 adds the block to its group's count.  exit_mid,
// once that count's old value has come back: the block that completed its
// group adds the group to the top count.  exit_final: the block that completed
// the top count clears every word.  A down block runs the first two in the
// middle of its work (right after its last wait and after staging h), so the
// round trips overlap its products.
__device__ __forceinline__ uint32_t exit_begin(uint32_t* sync) {
    uint32_t old = 0;
    if (threadIdx.x == 0) old = atomic_add_dev(sync_word(sync, SW_EXIT + (blockIdx.x & 7)), 1u);
    return old;
}
__device__ __forceinline__ uint32_t exit_mid(uint32_t* sync, uint32_t old) {
    uint32_t top = ~0u;
    if (threadIdx.x == 0) {
        const uint32_t g = blockIdx.x & 7;
        if (old == group_size(gridDim.x, g) - 1) {
            store_dev(sync_word(sync, SW_EXIT + g), 0u);   // the whole group has exited
            top = atomic_add_dev(sync_word(sync, SW_EXIT_TOP), 1u);
        }
    }
    return top;
}
__device__ __forceinline__ void exit_final(uint32_t* sync, uint32_t top) {
    if (threadIdx.x < WAVE) {
        const uint32_t groups = gridDim.x < 8 ? gridDim.x : 8;
        const uint32_t last = threadIdx.x == 0 && top == groups - 1;
        if (__shfl(last, 0, WAVE)) {   // every block is past its waits: clear the rest
            const int l = threadIdx.x;
            store_dev(sync_word(sync, FL_DONE + l), 0u);
#pragma unroll
            for (int q = 0; q < 4; ++q)   // the plan flag copy, record words included
                st_dev16(sync_word(sync, FL_PLAN + l) + 4 * q, 0u, 0u, 0u, 0u);
            store_dev(sync_word(sync, FL_VICT + l), 0u);
            if (l < 8) store_dev(sync_word(sync, SW_DONE + l), 0u);
            if (l == 0) {
                store_dev(sync_word(sync, SW_DONE_TOP), 0u);
                store_dev(sync_word(sync, SW_EXIT_TOP), 0u);
            }
        }
    }
}
__device__ __forceinline__ void block_exit(uint32_t* sync) {
    __syncthreads();
    exit_final(sync, exit_mid(sync, exit_begin(sync)));
}

// 16 bytes by two device-scope 8-byte loads.
__device__ __forceinline__ uint4 ld_dev16(const void* q) {
    const uint64_t* w = reinterpret_cast<const uint64_t*>(q);
    const uint64_t a = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t b = __hip_atomic_load(w + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_uint4(static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32),
                      static_cast<uint32_t>(b), static_cast<uint32_t>(b >> 32));
}

__device__ __forceinline__ int32_t ld_dev32(const int32_t* q) {
    return __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Whole-layer launch: the plan comes from the bookkeeping workgroup of the same
// launch, so it is read with device-scope loads once its flag is up.
__device__ __forceinline__ void stage_plan_dev(const DecodeParams& p, PlanLds& pl) {
    const int t = threadIdx.x;
    if (t < p.n_plan) {
        const uint4 r = ld_dev16(p.plan + 4 * t);
        pl.plan[t] = make_int4(static_cast<int>(r.x), static_cast<int>(r.y), static_cast<int>(r.z),
                               static_cast<int>(r.w));
        pl.uniq[t] = ld_dev32(p.uniq + t);
    }
    if (t < p.T * p.k) {
        const int32_t pr = ld_dev32(p.pairs + t);
        pl.pairs[t] = pr;
        pl.tok[t] = pr / p.k;
        pl.w[t] = __int_as_float(ld_dev32(reinterpret_cast<const int32_t*>(p.w) + t));
    }
    if (t == 0) pl.n_uniq = ld_dev32(p.counts);
    __syncthreads();
}

// Whole-layer launch, one-token plan record: until every word of copy b % 64 of
// the plan flag carries REC_BIT (lanes 0..3 poll 16 bytes each); the record
// then fills the staged plan (pair u of expert u, token 0).  The record is the
// first plan and never names the fills: a block that finds the victims flag
// already up (a block that starts late) stages the final plan from memory
// instead.  A wait that gives up stages no experts.
__device__ __forceinline__ void wait_plan_record(uint32_t* sync, uint32_t b, const DecodeParams& p,
                                                 PlanLds& pl) {
    const int t = threadIdx.x;
    if (t < 4) {
        const uint32_t* rec = sync_word(sync, FL_PLAN + static_cast<int>(b & 63));
        const uint32_t* vw = sync_word(sync, FL_VICT + static_cast<int>(b & 63));
        uint32_t n = 0, v = 0;
        bool whole = false;
        uint4 r;
        while (true) {
            if (t == 0) v = __hip_atomic_load(vw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            r = ld_dev16(rec + 4 * t);
            if (__shfl(v, 0, 4) != 0u) break;
            whole = (__ballot((r.x & r.y & r.z & r.w & REC_BIT) != 0u) & 0xFull) == 0xFull;
            if (whole) break;
            __builtin_amdgcn_s_sleep(2);
            if (++n == SPIN_LIMIT) {
                if (t == 0)
                    __hip_atomic_fetch_or(p.err, ERR_WAIT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
        pl.rec[4 * t] = r.x;
        pl.rec[4 * t + 1] = r.y;
        pl.rec[4 * t + 2] = r.z;
        pl.rec[4 * t + 3] = r.w;
        if (t == 0) {
            pl.fills_known = v != 0u;
            pl.n_uniq = whole ? p.k : 0;
        }
    }
    __syncthreads();
    if (pl.fills_known) {   // block-uniform
        stage_plan_dev(p, pl);
        return;
    }
    if (t < p.k && pl.n_uniq > 0) {
        const uint32_t a = pl.rec[t];
        const int pair = static_cast<int>(a & 63u);
        pl.plan[t] = make_int4((a >> 30) & 1u ? -1 : static_cast<int>((a >> 16) & 0x3FFFu), 0, t, 1);
        pl.uniq[t] = static_cast<int>((a >> 6) & 0x3FFu);
        pl.pairs[t] = pair;
        pl.tok[t] = 0;
        pl.w[pair] = __uint_as_float(pl.rec[REC_K + t] & ~REC_BIT);
    }
    __syncthreads();
}

// Whole-layer launch, a block that reads a missed expert (block-uniform `need`):
// wait until the fills' victim slots are published, then re-read the plan rows,
// which now name the slot each filled expert is written to.
__device__ __forceinline__ void refresh_for_fills(const DecodeParams& p, PlanLds& pl,
                                                  uint32_t* sync, bool need) {
    if (!need) return;
    wait_flag(sync, FL_VICT, blockIdx.x, p.err);
    if (threadIdx.x < p.n_plan) {
        const uint4 r = ld_dev16(p.plan + 4 * threadIdx.x);
        pl.plan[threadIdx.x] = make_int4(static_cast<int>(r.x), static_cast<int>(r.y),
                                         static_cast<int>(r.z), static_cast<int>(r.w));
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// gate/up.  KW wavefronts share a row tile and split H; RT tiles of 16 rows each.
template <int FMT, int KW, int RT>
struct GuStage {
    WSlab<RT> g, u;
    uint4 x[4];
};

// Position in a block's or wavefront's stream of stages: (item, token group, slab).
struct Cursor {
    int item, tg, s;
    bool valid;
};

// NW wavefronts per block (KW of them split H, NW / KW row groups); D stages in
// flight per wavefront.  SKIP: a wavefront's loads past its last stage are
// skipped instead of repeated (used when all of a wavefront's loads fit in the
// ring's first D - 1 stages, so nothing is lost by the compiler's coarser wait).
// The gate/up work of block `bid` of `nblk`.  WH: h leaves multiplied by its
// pair's routing weight (the fused small-call kernel sums experts in its down
// products) and written through to the device coherence point; otherwise the
// down pass applies the weight.
template <int FMT, int NW, int KW, int RT, int D, bool SKIP, bool WH>
__device__ __forceinline__ void gate_up_body(const DecodeParams& p, PlanLds& pl,
                                             f32x4 (&red)[SKIP ? 1 : 2][NW][RT][2][WAVE],
                                             int bid, int nblk, uint32_t* fill_sync = nullptr) {
    constexpr int RW = NW / KW;
    constexpr int NB = SKIP ? 1 : 2;   // reduction buffers (one item per block when SKIP)
    const int lane = threadIdx.x & (WAVE - 1), ln = lane & 15, gq = lane >> 4;
    const int wv = threadIdx.x / WAVE, kw = wv % KW, rw = wv / KW;
    const int H = p.H;
    const int kpart = H / KW, NS = kpart / SLAB, kbase = kw * kpart;
    const int tile_rows = RW * RT * 16;
    const int tiles = p.I / tile_rows;
    const int n_items = pl.n_uniq * tiles;
    // items bid, bid + nblk, ...: every block gets floor or ceil(n_items / nblk)
    // (contiguous ranges of ceil(n_items / nblk) left the last blocks empty,
    // and the CUs that held two full blocks set the time)
    const int i_beg = bid;
    if (i_beg >= n_items) return;
    const int i_last = i_beg + (n_items - 1 - i_beg) / nblk * nblk;

    // unit = (item, token group); stage = (unit, slab)
    auto tokens_of = [&](int item) { return pl.plan[item / tiles].w; };
    // Loads are unconditional so that the compiler can count the ones still in
    // flight: a cursor past the block's end re-reads its last item, and token
    // columns with no pair read the expert's first token (their MFMA columns are
    // never used).
    auto load = [&](GuStage<FMT, KW, RT>& st, int item, int tg, int s) {
        const int it = min(item, i_last);
        const int u = it / tiles, tile = it - u * tiles;
        const ExpertRef ref = expert_ref(p, pl, u);
        const int row0 = tile * tile_rows + rw * RT * 16;
        const int kb = kbase + s * SLAB;
        load_wslab<FMT, RT>(p, ref.src, 0, row0, H, kb, ln, gq, st.g);
        load_wslab<FMT, RT>(p, ref.src, 1, row0, H, kb, ln, gq, st.u);
        const int4 pr = pl.plan[u];
        const int n = tg * TOK + ln;
        // only lanes of a token column that holds a pair load x (the address
        // unit then sees a fraction of the lanes when an expert has few tokens);
        // the other columns are zero and their MFMA results are never read
        if (n < pr.w) {
            const int t = pl.tok[pr.z + n];
            // 32-bit offset from the (scalar) base: x is far below 4 GiB
            const uint16_t* xs = p.x + (static_cast<uint32_t>(t) * static_cast<uint32_t>(H) + static_cast<uint32_t>(kb + 32 * gq));
#pragma unroll
            for (int i = 0; i < 4; ++i) st.x[i] = ldg16(xs + 8 * i);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) st.x[i] = make_uint4(0u, 0u, 0u, 0u);
        }
    };
    f32x4 acc[2][RT];
    // int4: largest bf16 magnitude of x seen and whether an h value left f16's
    // range (either makes the f16 operands inexact: flagged in the error word)
    u16x2_t xmag = {0, 0};
    bool hbad = false;
    auto zero_acc = [&]() {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int t = 0; t < RT; ++t) acc[m][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    };
    auto compute = [&](const GuStage<FMT, KW, RT>& st, int item, int tg, int s) {
        uint4 b[4];
        float part = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            b[j] = FMT == MOE355_W_INT4_G64 ? b_x_f16(st.x[j], &part) : st.x[j];
            if (FMT == MOE355_W_INT4_G64) xmag = bf16_mag_max(st.x[j], xmag);
        }
        mma_slab<FMT, RT>(st.g, b, gq, acc[0]);
        mma_slab<FMT, RT>(st.u, b, gq, acc[1]);
        if (FMT == MOE355_W_INT4_G64) {
            const uint4 bb = bias_b_operand(part, gq);
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                acc[0][t] = mma<FMT>(bias_a_operand(st.g.bi[t], st.g.sc[t], gq), bb, acc[0][t]);
                acc[1][t] = mma<FMT>(bias_a_operand(st.u.bi[t], st.u.sc[t], gq), bb, acc[1][t]);
            }
        }
        if (tg == 0) {
            const int u = item / tiles;
            const ExpertRef ref = expert_ref(p, pl, u);
            if (ref.dst) {
                const int row0 = (item - u * tiles) * tile_rows + rw * RT * 16;
                const int kb = kbase + s * SLAB;
                store_wslab<FMT, RT>(p, ref.dst, 0, row0, H, kb, ln, gq, st.g);
                store_wslab<FMT, RT>(p, ref.dst, 1, row0, H, kb, ln, gq, st.u);
            }
        }
    };
    int ebuf = 0;
    auto epilogue = [&](int item, int tg) {
        const int u = item / tiles;
        const int4 pr = pl.plan[u];
        if (KW > 1) {
            if (kw != 0) {
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int t = 0; t < RT; ++t) red[ebuf][wv][t][m][lane] = acc[m][t];
            }
            __syncthreads();
            if (kw == 0) {
#pragma unroll
                for (int o = 1; o < KW; ++o)
#pragma unroll
                    for (int m = 0; m < 2; ++m)
#pragma unroll
                        for (int t = 0; t < RT; ++t) acc[m][t] += red[ebuf][wv + o][t][m][lane];
            }
            if (NB == 2) ebuf ^= 1;
        }
        const int n = tg * TOK + ln;
        if (WH && kw == 0 && n < pr.w) {
            // w * h of rows row0 + 16 t + 4 gq + 0..3 as one 16-byte piece (four hi
            // halves, then four lo halves, rows in natural order) per lane: the
            // four lanes of a token write 64 contiguous bytes, through to the
            // device coherence point
            const int pair = pl.pairs[pr.z + n];
            const float wt = pl.w[pair];
            const int row0 = (item - u * tiles) * tile_rows + rw * RT * 16;
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float hv = silu(acc[0][t][r]) * acc[1][t][r] * wt;
                    if (FMT == MOE355_W_INT4_G64) {
                        hbad |= beyond_f16(hv);
                        const _Float16 a = static_cast<_Float16>(hv);
                        const _Float16 b = static_cast<_Float16>(hv - static_cast<float>(a));
                        hi[r] = __builtin_bit_cast(uint16_t, a);
                        lo[r] = __builtin_bit_cast(uint16_t, b);
                    } else {
                        const __bf16 a = static_cast<__bf16>(hv);
                        const __bf16 b = static_cast<__bf16>(hv - static_cast<float>(a));
                        hi[r] = __builtin_bit_cast(uint16_t, a);
                        lo[r] = __builtin_bit_cast(uint16_t, b);
                    }
                }
                uint4* dst = reinterpret_cast<uint4*>(p.h_hi) +
                             (static_cast<int64_t>(pair) * p.I + row0 + 16 * t + 4 * gq) / 4;
                st_dev16(dst, hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), lo[0] | (lo[1] << 16),
                         lo[2] | (lo[3] << 16));
            }
        }
        if (!WH && kw == 0 && n < pr.w) {
            const int pair = pl.pairs[pr.z + n];
            const int row0 = (item - u * tiles) * tile_rows + rw * RT * 16;
#pragma unroll
            for (int t = 0; t < RT; ++t) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float hv = silu(acc[0][t][r]) * acc[1][t][r];
                    const int row = row0 + 16 * t + 4 * gq + r;
                    uint16_t hi, lo;
                    int64_t at;
                    if (FMT == MOE355_W_INT4_G64) {
                        hbad |= beyond_f16(hv);
                        const _Float16 a = static_cast<_Float16>(hv);
                        const _Float16 b = static_cast<_Float16>(hv - static_cast<float>(a));
                        hi = __builtin_bit_cast(uint16_t, a);
                        lo = __builtin_bit_cast(uint16_t, b);
                        // stored in the int4 A order inside each block of 8 rows
                        at = static_cast<int64_t>(pair) * p.I + (row & ~7) + 2 * r + (gq & 1);
                    } else {
                        const __bf16 a = static_cast<__bf16>(hv);
                        const __bf16 b = static_cast<__bf16>(hv - static_cast<float>(a));
                        hi = __builtin_bit_cast(uint16_t, a);
                        lo = __builtin_bit_cast(uint16_t, b);
                        at = static_cast<int64_t>(pair) * p.I + row;
                    }
                    p.h_hi[at] = hi;
                    p.h_lo[at] = lo;
                }
            }
        }
        zero_acc();
    };

    zero_acc();
    auto advance = [&](Cursor& c) {
        if (!c.valid) return;
        if (++c.s < NS) return;
        c.s = 0;
        if ((c.tg + 1) * TOK < tokens_of(c.item)) {
            ++c.tg;
            return;
        }
        c.tg = 0;
        c.item += nblk;
        c.valid = c.item <= i_last;
    };
    // D stages in a ring: the loads of the next D-1 stages stay in flight while
    // one is computed
    GuStage<FMT, KW, RT> st[D];
    Cursor lc{i_beg, 0, 0, true}, cc = lc;
#pragma unroll
    for (int d = 0; d < D - 1; ++d) {
        if (!SKIP || lc.valid) load(st[d], lc.item, lc.tg, lc.s);
        advance(lc);
    }
    // Without SKIP every step of the unrolled ring issues its loads (a cursor
    // past the end re-reads its last item) and only the computation is
    // guarded: a guarded load lets the compiler's wait before a stage's MFMAs
    // count only the loads present on every path (one stage of lookahead).
    // whole-layer launch: a block reading a missed expert learns where to write
    // it (the fills' victim slots) before its first fill-through store
    bool fresh = fill_sync == nullptr;
    bool need = false;
    if (!fresh)
        for (int it = i_beg; it <= i_last; it += nblk) need |= pl.plan[it / tiles].x < 0;
    bool done = false;
    while (!done) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (!SKIP || lc.valid) load(st[(d + D - 1) % D], lc.item, lc.tg, lc.s);
            advance(lc);
            if (!done) {
                if (!fresh) {
                    refresh_for_fills(p, pl, fill_sync, need);
                    fresh = true;
                }
                compute(st[d], cc.item, cc.tg, cc.s);
                if (cc.s == NS - 1) epilogue(cc.item, cc.tg);
                advance(cc);
                done = !cc.valid;
            }
        }
    }
    if (FMT == MOE355_W_INT4_G64 && (hbad || bf16_mag_beyond_f16(xmag)))
        __hip_atomic_fetch_or(p.err, ERR_F16_RANGE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int FMT, int NW, int KW, int RT, int D, bool SKIP>
__global__ void __launch_bounds__(NW * WAVE) gate_up_kernel(DecodeParams p) {
    __shared__ PlanLds pl;
    __shared__ f32x4 red[SKIP ? 1 : 2][NW][RT][2][WAVE];
    stage_plan(p, pl);
    {   // zero the layer output for the down launch's atomics
        const int64_t n = static_cast<int64_t>(p.T) * p.H;
        for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
             i += static_cast<int64_t>(gridDim.x) * blockDim.x)
            p.out[i] = 0.0f;
    }
    gate_up_body<FMT, NW, KW, RT, D, SKIP, false>(p, pl, red, blockIdx.x, gridDim.x);
}

// ---------------------------------------------------------------------------
// down + combine.  Wavefront items of RT tiles of 16 rows over all of I.
template <int FMT, int RT>
struct DnStage {
    WSlab<RT> w;
    uint4 hh[4], hl[4];
};

// KSPLIT wavefronts share a row tile and split I (their partial sums meet in the
// output atomics); SKIP as in the gate/up kernel.
template <int FMT, int RT, int D, int KSPLIT, bool SKIP>
__global__ void __launch_bounds__(256) down_kernel(DecodeParams p) {
    __shared__ PlanLds pl;
    const int lane = threadIdx.x & (WAVE - 1), ln = lane & 15, gq = lane >> 4;
    stage_plan(p, pl);
    const int I = p.I, NS = I / SLAB / KSPLIT;
    const int tile_rows = RT * 16;
    const int tiles = p.H / tile_rows;
    const int n_items = pl.n_uniq * tiles * KSPLIT;
    const int n_waves = gridDim.x * (blockDim.x / WAVE);
    const int gw = blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE;
    const int per = (n_items + n_waves - 1) / n_waves;
    const int i_beg = gw * per;
    const int i_end = min(n_items, i_beg + per);
    if (i_beg >= i_end) return;

    // item = (distinct expert u, row tile, part ks of I)
    const int per_u = tiles * KSPLIT;
    auto tokens_of = [&](int item) { return pl.plan[item / per_u].w; };
    auto kbase_of = [&](int item) { return (item % KSPLIT) * (I / KSPLIT); };
    auto tile_of = [&](int item) { return (item % per_u) / KSPLIT; };
    // unconditional loads (unless SKIP), as in gate/up
    auto load = [&](DnStage<FMT, RT>& st, int item, int tg, int s) {
        const int it = min(item, i_end - 1);
        const int u = it / per_u, tile = tile_of(it);
        const ExpertRef ref = expert_ref(p, pl, u);
        const int kb = kbase_of(it) + s * SLAB;
        load_wslab<FMT, RT>(p, ref.src, 2, tile * tile_rows, I, kb, ln, gq, st.w);
        const int4 pr = pl.plan[u];
        const int n = tg * TOK + ln;
        if (n < pr.w) {   // as in gate/up: only columns holding a pair load h
            const uint32_t o = static_cast<uint32_t>(pl.pairs[pr.z + n]) * static_cast<uint32_t>(I) +
                               static_cast<uint32_t>(kb + 32 * gq);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                st.hh[i] = ldg16(p.h_hi + o + 8 * i);
                st.hl[i] = ldg16(p.h_lo + o + 8 * i);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) st.hh[i] = st.hl[i] = make_uint4(0u, 0u, 0u, 0u);
        }
    };
    f32x4 acc[RT];
    auto zero_acc = [&]() {
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    };
    auto compute = [&](const DnStage<FMT, RT>& st, int item, int tg, int s) {
        mma_slab2<FMT, RT>(st.w, st.hh, st.hl, gq, acc);
        if (FMT == MOE355_W_INT4_G64) {
            float part = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) part = sum_f16x8(st.hl[i], sum_f16x8(st.hh[i], part));
            const uint4 bb = bias_b_operand(part, gq);
#pragma unroll
            for (int t = 0; t < RT; ++t)
                acc[t] = mma<FMT>(bias_a_operand(st.w.bi[t], st.w.sc[t], gq), bb, acc[t]);
        }
        if (tg == 0) {
            const ExpertRef ref = expert_ref(p, pl, item / per_u);
            if (ref.dst)
                store_wslab<FMT, RT>(p, ref.dst, 2, tile_of(item) * tile_rows, I,
                                     kbase_of(item) + s * SLAB, ln, gq, st.w);
        }
    };
    auto epilogue = [&](int item, int tg) {
        const int u = item / per_u;
        const int4 pr = pl.plan[u];
        const int n = tg * TOK + ln;
        if (n < pr.w) {
            const int pair = pl.pairs[pr.z + n];
            const float wt = pl.w[pair];
            float* o = p.out + static_cast<int64_t>(pl.tok[pr.z + n]) * p.H + tile_of(item) * tile_rows;
#pragma unroll
            for (int t = 0; t < RT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) unsafeAtomicAdd(o + 16 * t + 4 * gq + r, wt * acc[t][r]);
        }
        zero_acc();
    };

    zero_acc();
    auto advance = [&](Cursor& c) {
        if (!c.valid) return;
        if (++c.s < NS) return;
        c.s = 0;
        if ((c.tg + 1) * TOK < tokens_of(c.item)) {
            ++c.tg;
            return;
        }
        c.tg = 0;
        c.valid = ++c.item < i_end;
    };
    // D stages in a ring: the loads of the next D-1 stages stay in flight while
    // one is computed
    DnStage<FMT, RT> st[D];
    Cursor lc{i_beg, 0, 0, true}, cc = lc;
#pragma unroll
    for (int d = 0; d < D - 1; ++d) {
        if (!SKIP || lc.valid) load(st[d], lc.item, lc.tg, lc.s);
        advance(lc);
    }
    // Without SKIP every step of the unrolled ring issues its loads (a cursor
    // past the end re-reads its last item) and only the computation is
    // guarded: a guarded load lets the compiler's wait before a stage's MFMAs
    // count only the loads present on every path (one stage of lookahead).
    bool done = false;
    while (!done) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (!SKIP || lc.valid) load(st[(d + D - 1) % D], lc.item, lc.tg, lc.s);
            advance(lc);
            if (!done) {
                compute(st[d], cc.item, cc.tg, cc.s);
                if (cc.s == NS - 1) epilogue(cc.item, cc.tg);
                advance(cc);
                done = !cc.valid;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// down + combine with h in LDS (many distinct experts, e.g. the DS-like decode).
// The work is cut into units (distinct expert u, token group tg of up to 16 of
// its pairs, 16 RT consecutive output rows), each computed over all of I by one
// wavefront (RT 16-row tiles); a block of NW wavefronts takes a contiguous,
// balanced range of units.  The block keeps the h rows (hi and lo halves) of a
// window of consecutive pair positions in LDS, staged before its first unit and
// again only when a unit's pairs leave the window (the positions of
// consecutive units rise), so a wavefront's register ring holds weights alone
// and runs D - 1 slabs ahead.  (With h in the ring, each
// stage also held 32 registers of h and two stages ahead filled the register
// budget at two wavefronts per SIMD: half the bytes in flight of gate/up.)
constexpr int DNL_LDS = 135168;   // bytes of staged h: 16 rows of I = 2048 with padding

// NW wavefronts per block, one block per CU
template <int FMT, int RT, int D, int NW>
__global__ void __launch_bounds__(NW * WAVE) down_lds_kernel(DecodeParams p) {
    __shared__ PlanLds pl;
    __shared__ int32_t tgb[MAX_PLAN + 1];   // item base of each distinct expert, in token groups
    __shared__ int32_t win[2];              // staged pair positions [win[0], win[1])
    __shared__ uint4 hsm[DNL_LDS / 16];
    stage_plan(p, pl);
    const int lane = threadIdx.x & (WAVE - 1), ln = lane & 15, gq = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);   // cursors in scalar registers
    constexpr int WR = 16 * RT;   // output rows per wavefront
    const int I = p.I, NS = I / SLAB;
    // row r of the window: hi halves (I / 8 uint4), lo halves, one uint4 of padding
    // (consecutive rows then start 4 banks apart, so 16 token rows do not collide)
    const int RSq = I / 4 + 1;
    const int nwin = min(DNL_LDS / 16 / RSq, 64);
    const int nu = pl.n_uniq;
    if (nu <= 0) return;
    if (threadIdx.x == 0) {
        int acc = 0;
        for (int u = 0; u < nu; ++u) {
            tgb[u] = acc;
            acc += max(1, (pl.plan[u].w + TOK - 1) / TOK);
        }
        tgb[nu] = acc;
    }
    __syncthreads();
    // Units of WR rows: unit j = (token group q = j / NB, row band j % NB).  Block
    // b owns units [jb, je) of a balanced split (one unit more or less than
    // any other block), so a call with fewer 1024-row chunks than blocks still
    // spreads its bytes over every CU; wavefront w takes units jb + w + NW i.
    // A block's units visit the token groups q_first .. q_last in phases: a
    // phase's units multiply the h rows of their group, which the window holds
    // (it is restaged, between two barriers, only when a phase's group is
    // outside it; every wavefront takes part in every phase change, including
    // those of phases in which it has no unit).
    const int NB = p.H / WR;
    const int n_units = tgb[nu] * NB;
    const int nb = static_cast<int>(gridDim.x), b = static_cast<int>(blockIdx.x);
    const int jb = static_cast<int>(static_cast<int64_t>(n_units) * b / nb);
    const int je = static_cast<int>(static_cast<int64_t>(n_units) * (b + 1) / nb);
    if (jb >= je) return;   // block-uniform
    const int q_first = jb / NB, q_last = (je - 1) / NB;

    // cursor over the wavefront's (unit, slab) sequence; past its last unit it
    // re-reads that unit's last slab
    struct Cur {
        int j, s, u, tg, band;
        bool valid;
    };
    auto locate = [&](Cur& k, int j) {
        k.j = j;
        const int q = j / NB;
        k.band = j - q * NB;
        int lo = 0, hi = nu - 1;   // the last u with tgb[u] <= q
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tgb[mid] <= q) lo = mid;
            else hi = mid - 1;
        }
        k.u = lo;
        k.tg = q - tgb[lo];
    };
    auto first = [&](Cur& k) {
        k.s = 0;
        k.valid = jb + wv < je;
        locate(k, k.valid ? jb + wv : je - 1);
    };
    auto adv = [&](Cur& k) {
        if (++k.s < NS) return;
        if (k.valid && k.j + NW < je) {
            k.s = 0;
            locate(k, k.j + NW);
        } else {
            k.valid = false;
            k.s = NS - 1;
        }
    };
    auto q_of = [&](const Cur& k) { return k.j / NB; };
    // pair positions of token group q: [a, a + nt)
    auto group_at = [&](int q, int& a, int& nt) {
        int lo = 0, hi = nu - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tgb[mid] <= q) lo = mid;
            else hi = mid - 1;
        }
        const int4 pr = pl.plan[lo];
        const int tg = q - tgb[lo];
        a = pr.z + TOK * tg;
        nt = min(TOK, pr.w - TOK * tg);
    };
    // pair positions this block's units use end at its last group
    int n_pos;
    {
        int a, nt;
        group_at(q_last, a, nt);
        n_pos = a + nt;
    }
    // the window from pair position p0 on (all threads; ends with a barrier)
    auto stage_h = [&](int p0) {
        const int nr = min(nwin, n_pos - p0);
        const int rq = I / 4;   // uint4 of h per row
        const int n = nr * rq;
        // eight loads in flight per thread before their LDS stores (one load,
        // wait and store at a time made the window a chain of round trips)
        constexpr int B = 8;
        for (int i0 = threadIdx.x; i0 < n; i0 += B * NW * WAVE) {
            uint4 v[B];
            // without branches, so the compiler cannot sink each load next to its
            // store: chunks past the window re-read and rewrite chunk 0 (the same
            // value)
            int at[B];
#pragma unroll
            for (int j = 0; j < B; ++j) {
                const int i = i0 + j * NW * WAVE < n ? i0 + j * NW * WAVE : 0;
                const int r = i / rq, c = i - r * rq;
                const int64_t pair = pl.pairs[p0 + r];
                const uint16_t* base = c < I / 8 ? p.h_hi : p.h_lo;
                v[j] = reinterpret_cast<const uint4*>(base + pair * I)[c < I / 8 ? c : c - I / 8];
                at[j] = r * RSq + c;
            }
#pragma unroll
            for (int j = 0; j < B; ++j) hsm[at[j]] = v[j];
        }
        if (threadIdx.x == 0) {
            win[0] = p0;
            win[1] = p0 + nr;
        }
        __syncthreads();
    };
    // phase change to group q (every wavefront, in phase order)
    auto enter = [&](int q) {
        int a, nt;
        group_at(q, a, nt);
        if (a < win[0] || a + nt > win[1]) {   // block-uniform
            __syncthreads();   // every wavefront is done with the old window
            stage_h(a);
        }
    };
    auto group_of = [&](const Cur& k, int& a, int& nt) {
        const int4 pr = pl.plan[k.u];
        a = pr.z + TOK * k.tg;
        nt = min(TOK, pr.w - TOK * k.tg);
    };

    f32x4 acc[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    auto load_stage = [&](WSlab<RT>& w, const Cur& k) {
        const ExpertRef ref = expert_ref(p, pl, k.u);
        load_wslab<FMT, RT>(p, ref.src, 2, k.band * WR, I, k.s * SLAB, ln, gq, w);
    };
    auto compute = [&](const WSlab<RT>& w, const Cur& k) {
        int a, nt;
        group_of(k, a, nt);
        uint4 hh[4], hl[4];
        if (ln < nt) {
            const uint4* row = hsm + (a + ln - win[0]) * RSq + k.s * (SLAB / 8) + 4 * gq;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                hh[i] = row[i];
                hl[i] = row[I / 8 + i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) hh[i] = hl[i] = make_uint4(0u, 0u, 0u, 0u);
        }
        mma_slab2<FMT, RT>(w, hh, hl, gq, acc);
        if (FMT == MOE355_W_INT4_G64) {
            float part = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) part = sum_f16x8(hl[i], sum_f16x8(hh[i], part));
            const uint4 bb = bias_b_operand(part, gq);
#pragma unroll
            for (int t = 0; t < RT; ++t) acc[t] = mma<FMT>(bias_a_operand(w.bi[t], w.sc[t], gq), bb, acc[t]);
        }
        if (k.tg == 0) {   // fill-through of the expert's down bytes
            const ExpertRef ref = expert_ref(p, pl, k.u);
            if (ref.dst) store_wslab<FMT, RT>(p, ref.dst, 2, k.band * WR, I, k.s * SLAB, ln, gq, w);
        }
    };
    auto epilogue = [&](const Cur& k) {
        int a, nt;
        group_of(k, a, nt);
        if (ln < nt) {
            const int pair = pl.pairs[a + ln];
            const float wt = pl.w[pair];
            float* o = p.out + static_cast<int64_t>(pl.tok[a + ln]) * p.H + k.band * WR;
#pragma unroll
            for (int t = 0; t < RT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) unsafeAtomicAdd(o + 16 * t + 4 * gq + r, wt * acc[t][r]);
        }
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    };

    Cur lc, cc;
    first(lc);
    cc = lc;
    // the first weight stages do not depend on h: their loads go out before the
    // window is staged
    WSlab<RT> ring[D];
    if (cc.valid) {
#pragma unroll
        for (int d = 0; d < D - 1; ++d) {
            load_stage(ring[d], lc);
            adv(lc);
        }
    }
    {
        int a, nt;
        group_at(q_first, a, nt);
        stage_h(a);
    }
    int cur_q = q_first;   // the phase every wavefront has entered
    bool done = !cc.valid;
    while (!done) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            load_stage(ring[(d + D - 1) % D], lc);
            adv(lc);
            if (!done) {
                if (cc.s == 0)
                    while (cur_q < q_of(cc)) enter(++cur_q);
                compute(ring[d], cc);
                if (cc.s == NS - 1) epilogue(cc);
                adv(cc);
                done = !cc.valid;
            }
        }
    }
    while (cur_q < q_last) enter(++cur_q);   // the phases of the other wavefronts' units
}

// ---------------------------------------------------------------------------
// Fused small-call FFN: one launch in which blocks [0, G) run the gate/up work
// (h leaves multiplied by the routing weight; they also zero the output) and
// blocks [G, G + 2 H/16) come in pairs that own 16 output rows of every token:
// each sums the down products of half of the distinct experts' slabs and adds
// its result onto the output.  A down block loads and dequantises its weights at
// once (they do not depend on h), then waits until all G gate/up blocks have
// counted themselves done, stages the call's h in LDS and runs its products.
//
// Waits only ever point at lower block indices and a gate/up block never waits,
// so the call finishes whatever the number of resident blocks: every XCD
// dispatches its blocks in index order.  Every wait is also bounded (it gives
// up, flags the error word and goes on) so that a block always exits.
//

constexpr int SMALL_DB = 2;            // (expert, slab) items per down wavefront
constexpr int SMALL_H_LDS = 32768;     // bytes of h (hi and lo halves of T*k*I values) in LDS

// One slab's weights as MFMA A operands (and, for int4, the bias operand).
struct ASlab {
    uint4 a[4];
    uint4 bias;
};
template <int FMT>
__device__ __forceinline__ ASlab prep_a(const WSlab<1>& w, int gq) {
    ASlab r;
    const uint32_t d4[4] = {w.q[0].x, w.q[0].y, w.q[0].z, w.q[0].w};
    if (FMT == MOE355_W_INT4_G64) {
        const half2_t s2 = int4_scale(w.sc[0], gq);
#pragma unroll
        for (int j = 0; j < 4; ++j) r.a[j] = a_int4(d4[j], s2);
        r.bias = bias_a_operand(w.bi[0], w.sc[0], gq);
    } else {
        const float scale = e8m0_to_f32((w.sc[0] >> (8 * gq)) & 0xFFu);
#pragma unroll
        for (int j = 0; j < 4; ++j) r.a[j] = a_fp4(d4[j], scale);
        r.bias = make_uint4(0u, 0u, 0u, 0u);
    }
    return r;
}

// Down rows r0 .. r0+15 of every token, half `half` of the (distinct expert u,
// 128-input slab) items: item 2 (wv + NW i) + half for i < SMALL_DB.  The B
// operand's column n is token n (T <= 16), holding that token's weighted h for
// u, or zero when the token is not routed to u.  The weights are loaded and
// dequantised before the wait; the wavefronts' partial sums meet through LDS
// and the two halves meet in fp32 atomic additions onto the zeroed output
// (0 + a + b in either order gives the same sum).
template <int FMT, int NW>
__device__ __forceinline__ void down_rows_body(const DecodeParams& p, PlanLds& pl,
                                               uint4* hs, f32x4 (&red)[NW][WAVE], int r0,
                                               int half, uint32_t* sync, uint32_t n_gu,
                                               bool layer_fills, uint32_t& exit_top) {
    const int lane = threadIdx.x & (WAVE - 1), ln = lane & 15, gq = lane >> 4;
    const int wv = threadIdx.x / WAVE;
    const int I = p.I, nsl = I / SLAB;
    const int n_items = pl.n_uniq * nsl;
    auto item_of = [&](int i) { return 2 * (wv + i * NW) + half; };
    // weights (unconditional: an item past the end re-reads the last one)
    WSlab<1> w[SMALL_DB];
    auto load_weights = [&]() {
        if (n_items > 0) {
#pragma unroll
            for (int i = 0; i < SMALL_DB; ++i) {
                const int j = min(item_of(i), n_items - 1);
                const int u = j / nsl, sl = j - u * nsl;
                load_wslab<FMT, 1>(p, expert_ref(p, pl, u).src, 2, r0, I, sl * SLAB, ln, gq, w[i]);
            }
        }
    };
    // alone, the down weights load at once (they do not depend on h); in the
    // whole-layer launch they load once the fills are known, which leaves the
    // memory system to the gate/up blocks' weights first
    if (!layer_fills) load_weights();
    auto fill_stores = [&]() {   // fill-through of this block's down bytes
#pragma unroll
        for (int i = 0; i < SMALL_DB; ++i) {
            const int j = item_of(i);
            if (j < n_items) {
                const int u = j / nsl;
                const ExpertRef ref = expert_ref(p, pl, u);
                if (ref.dst) store_wslab<FMT, 1>(p, ref.dst, 2, r0, I, (j - u * nsl) * SLAB, ln, gq, w[i]);
            }
        }
    };
    if (!layer_fills) fill_stores();
    if (layer_fills) {
        // whole-layer launch: once the fills' victim slots are published (while
        // the gate/up blocks compute), load, and write the filled experts' down
        // bytes to their slots
        bool need = false;   // block-uniform: over every wavefront's items
        for (int m = 0; m < NW * SMALL_DB; ++m) {
            const int j = 2 * m + half;
            if (j < n_items) need |= pl.plan[j / nsl].x < 0 || pl.plan[j / nsl].y != 0;
        }
        refresh_for_fills(p, pl, sync, need);
        load_weights();
        fill_stores();
    }
    ASlab A[SMALL_DB];
    int hoff[SMALL_DB];   // LDS piece of the lane's h for each item, or -1 (token not routed)
#pragma unroll
    for (int i = 0; i < SMALL_DB; ++i) {
        A[i] = prep_a<FMT>(w[i], gq);
        const int j = item_of(i);
        hoff[i] = -1;
        if (j < n_items) {
            const int u = j / nsl, sl = j - u * nsl;
            const int4 pr = pl.plan[u];
            for (int n = 0; n < pr.w; ++n)
                if (pl.tok[pr.z + n] == ln) hoff[i] = (pl.pairs[pr.z + n] * I + sl * SLAB + 32 * gq) / 4;
        }
    }
    wait_flag(sync, FL_DONE, blockIdx.x, p.err);
    const uint32_t exit_old = exit_begin(sync);   // no sync word is read after this wait
    // h pieces: [pair][I / 4] x 16 bytes (four hi halves, then four lo halves)
    const int nc = p.T * p.k * I / 4;
    {   // stage every pair's h in LDS: at most four pieces per thread
        static_assert(SMALL_H_LDS / 16 <= 4 * NW * WAVE, "h staging covers four pieces per thread");
        constexpr int NT = NW * WAVE;
        const int t0 = threadIdx.x;
        uint4 a0, a1, a2, a3;
        if (t0 < nc) a0 = ld_dev16(reinterpret_cast<const uint4*>(p.h_hi) + t0);
        if (t0 + NT < nc) a1 = ld_dev16(reinterpret_cast<const uint4*>(p.h_hi) + t0 + NT);
        if (t0 + 2 * NT < nc) a2 = ld_dev16(reinterpret_cast<const uint4*>(p.h_hi) + t0 + 2 * NT);
        if (t0 + 3 * NT < nc) a3 = ld_dev16(reinterpret_cast<const uint4*>(p.h_hi) + t0 + 3 * NT);
        if (t0 < nc) hs[t0] = a0;
        if (t0 + NT < nc) hs[t0 + NT] = a1;
        if (t0 + 2 * NT < nc) hs[t0 + 2 * NT] = a2;
        if (t0 + 3 * NT < nc) hs[t0 + 3 * NT] = a3;
        __syncthreads();
    }
    exit_top = exit_mid(sync, exit_old);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f}, acc_lo = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < SMALL_DB; ++i) {
        if (item_of(i) >= n_items) break;
        // B operands of the lane's 32 inputs sl * 128 + 32 gq + 8 q + (0..7): hi and
        // lo halves, in the int4 A order (0,4,1,5,2,6,3,7) or, for MXFP4, natural
        uint4 hh[4], hl[4];
        if (hoff[i] >= 0) {
            const uint4* src = hs + hoff[i];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 a = src[2 * q], b = src[2 * q + 1];   // inputs 0..3, 4..7
                if (FMT == MOE355_W_INT4_G64) {
                    hh[q] = make_uint4(__builtin_amdgcn_perm(b.x, a.x, 0x05040100u), __builtin_amdgcn_perm(b.x, a.x, 0x07060302u),
                                       __builtin_amdgcn_perm(b.y, a.y, 0x05040100u), __builtin_amdgcn_perm(b.y, a.y, 0x07060302u));
                    hl[q] = make_uint4(__builtin_amdgcn_perm(b.z, a.z, 0x05040100u), __builtin_amdgcn_perm(b.z, a.z, 0x07060302u),
                                       __builtin_amdgcn_perm(b.w, a.w, 0x05040100u), __builtin_amdgcn_perm(b.w, a.w, 0x07060302u));
                } else {
                    hh[q] = make_uint4(a.x, a.y, b.x, b.y);
                    hl[q] = make_uint4(a.z, a.w, b.z, b.w);
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) hh[q] = hl[q] = make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc = mma<FMT>(A[i].a[q], hh[q], acc);
            acc_lo = mma<FMT>(A[i].a[q], hl[q], acc_lo);
        }
        if (FMT == MOE355_W_INT4_G64) {
            float part[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) part[q] = sum_f16x8(hl[q], sum_f16x8(hh[q], 0.0f));
            acc = mma<FMT>(A[i].bias, bias_b_operand((part[0] + part[1]) + (part[2] + part[3]), gq), acc);
        }
    }
    acc += acc_lo;
    red[wv][lane] = acc;
    __syncthreads();
    if (wv == 0) {
#pragma unroll
        for (int o = 1; o < NW; ++o) acc += red[o][lane];
        if (ln < p.T) {
            float* o = p.out + static_cast<int64_t>(ln) * p.H + r0 + 4 * gq;
#pragma unroll
            for (int r = 0; r < 4; ++r) unsafeAtomicAdd(o + r, acc[r]);
        }
    }
}

template <int FMT, int NW, int D>
__global__ void __launch_bounds__(NW * WAVE, 4) ffn_small_kernel(DecodeParams p, uint32_t n_gu,
                                                              uint32_t* sync) {
    __shared__ PlanLds pl;
    // the gate/up reduction buffers, or the staged h and the down reduction
    constexpr int GU_BYTES = NW * 2 * WAVE * 16;
    constexpr int DN_BYTES = SMALL_H_LDS + NW * WAVE * 16;
    __shared__ uint4 raw[(GU_BYTES > DN_BYTES ? GU_BYTES : DN_BYTES) / 16];
    stage_plan(p, pl);
    if (blockIdx.x < n_gu) {
        {   // zero the output for the down blocks' additions (written through, and
            // complete before this block counts itself done)
            const int n = p.T * p.H;
            uint32_t* o = reinterpret_cast<uint32_t*>(p.out);
            for (int i = blockIdx.x * (NW * WAVE) + threadIdx.x; i < n; i += n_gu * (NW * WAVE))
                store_dev(o + i, 0u);
        }
        gate_up_body<FMT, NW, NW, 1, D, true, true>(
            p, pl, *reinterpret_cast<f32x4 (*)[1][NW][1][2][WAVE]>(raw), blockIdx.x, n_gu);
        signal_done(sync, n_gu, blockIdx.x);
    } else {
        const int b = blockIdx.x - n_gu;   // two blocks per 16-row tile
        uint32_t old;
        down_rows_body<FMT, NW>(p, pl, raw,
                                *reinterpret_cast<f32x4 (*)[NW][WAVE]>(raw + SMALL_H_LDS / 16),
                                (b >> 1) * 16, b & 1, sync, n_gu, false, old);
        exit_final(sync, old);
        return;
    }
    block_exit(sync);
}

bool valid_row_len(int L) {
    return L == 128 || L == 256 || L == 512 || L == 1024 || L == 2048 || L == 4096;
}

int device_cus() {
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        hipDeviceProp_t prop;
        if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess &&
            prop.multiProcessorCount > 0)
            cus = prop.multiProcessorCount;
        else
            cus = 256;
    }
    return cus;
}

template <int FMT, int KW>
moe355_status launch_gate_up(const DecodeParams& p, int max_uniq, hipStream_t stream) {
    constexpr int RW = 4 / KW;
    const int cap = device_cus() * 2;   // two resident blocks per CU
    // the widest tile that still leaves two items per block slot: four row tiles
    // per wavefront with two stages in flight (8 KB of gate and up codes per
    // stage; three when the call also writes fill-through bytes, which then run
    // at one wavefront per SIMD but keep more reads in flight beside the
    // stores), else two tiles with three stages, else one tile with four
    const int items2 = max_uniq * (p.I / (RW * 32));
    const int items4 = max_uniq * (p.I / (RW * 64));
    if (items4 >= 2 * cap && p.I % (RW * 64) == 0 && p.has_cache && p.fill_through) {
        gate_up_kernel<FMT, 4, KW, 4, 3, false><<<items4 < cap ? items4 : cap, 256, 0, stream>>>(p);
    } else if (items4 >= 2 * cap && p.I % (RW * 64) == 0) {
        gate_up_kernel<FMT, 4, KW, 4, 2, false><<<items4 < cap ? items4 : cap, 256, 0, stream>>>(p);
    } else if (items2 >= 2 * cap && p.I % (RW * 32) == 0) {
        gate_up_kernel<FMT, 4, KW, 2, 3, false><<<items2 < cap ? items2 : cap, 256, 0, stream>>>(p);
    } else {
        const int items1 = max_uniq * (p.I / (RW * 16));
        gate_up_kernel<FMT, 4, KW, 1, 4, false><<<items1 < cap ? items1 : cap, 256, 0, stream>>>(p);
    }
    return check_launch("expert_ffn_decode gate_up");
}

// Little work (a block per CU or fewer): eight wavefronts per block split H, so
// that two wavefronts per SIMD overlap their load and dequantisation chains;
// each wavefront's few slabs are all in flight at once.
template <int FMT>
moe355_status launch_gate_up_wide(const DecodeParams& p, int max_uniq, hipStream_t stream) {
    const int blocks = max_uniq * (p.I / 16);
    switch (p.H) {   // H / KW = 128 or 256 inputs per wavefront
        case 1024: gate_up_kernel<FMT, 8, 8, 1, 2, true><<<blocks, 512, 0, stream>>>(p); break;
        case 2048: gate_up_kernel<FMT, 16, 16, 1, 2, true><<<blocks, 1024, 0, stream>>>(p); break;
        default: gate_up_kernel<FMT, 16, 16, 1, 3, true><<<blocks, 1024, 0, stream>>>(p); break;
    }
    return check_launch("expert_ffn_decode gate_up");
}

// Whole-layer launch, after a gate/up block has counted itself done: once the
// fills' victim slots are published, the block copies its share of each filled
// expert's gate and up matrices (its 16-row tiles: contiguous code, scale and
// bias ranges in the device layout) from the pool to the slot.  The bytes were
// read moments ago, so the copy mostly hits the caches; it is off the path to
// the output.
template <int FMT>
__device__ __forceinline__ void copy_gate_up_fills(const DecodeParams& p, PlanLds& pl,
                                                   uint32_t* sync, int b, int n_gu) {
    const int tiles = p.I / 16;
    const int n_items = pl.n_uniq * tiles;
    const int per = (n_items + n_gu - 1) / n_gu;
    const int i_beg = b * per, i_end = min(n_items, i_beg + per);
    // block-uniform: a miss in the first plan, or a row already refreshed to a
    // fill (this block may have refreshed its plan in an earlier step)
    bool need = false;
    for (int it = i_beg; it < i_end; ++it) {
        const int4 row = pl.plan[it / tiles];
        need |= row.x < 0 || row.y != 0;
    }
    if (!need) return;
    refresh_for_fills(p, pl, sync, true);
    const uint32_t kb = static_cast<uint32_t>(p.H / 128);   // 128-input blocks per row tile
    for (int it = i_beg; it < i_end; ++it) {
        const int u = it / tiles, tile = it - u * tiles;
        const int4 row = pl.plan[u];
        if (!(row.x >= 0 && row.y)) continue;   // block-uniform
        const uint8_t* src = p.pool + (static_cast<int64_t>(p.layer) * p.E + pl.uniq[u]) * p.S;
        uint8_t* dst = const_cast<uint8_t*>(p.slots) + static_cast<int64_t>(row.x) * p.S;
        for (int m = 0; m < 2; ++m) {
            // (offset, bytes) of the tile's codes, scale words and bias words
            const uint32_t q0 = static_cast<uint32_t>(p.q_off[m]) + tile * kb * 1024u, qn = kb * 1024u;
            const uint32_t s0 = static_cast<uint32_t>(p.s_off[m]) + tile * kb * 64u, sn = kb * 64u;
            const uint32_t b0 = static_cast<uint32_t>(p.b_off[m]) + tile * kb * 64u;
            const uint32_t bn = FMT == MOE355_W_INT4_G64 ? kb * 64u : 0u;
            const uint32_t n16 = (qn + sn + bn) / 16;
            for (uint32_t c = threadIdx.x; c < n16; c += blockDim.x) {
                const uint32_t o = 16 * c;
                const uint32_t at = o < qn ? q0 + o : (o < qn + sn ? s0 + (o - qn) : b0 + (o - qn - sn));
                const uint4 v = *reinterpret_cast<const uint4*>(src + at);
                __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(dst + at));
            }
        }
    }
}

// Whole decode layer call in one launch: workgroup 0 runs the bookkeeping
// (routing, dedup, hit/miss, victims, slot update; classify_dev.h) and
// publishes the plan as soon as hits and misses are known; the other
// workgroups are the small-call FFN's gate/up and down blocks, which wait for
// that plan, stage it, and start streaming weights while workgroup 0 is still
// picking victims (a one-token call's plan travels as a record in the flag
// itself).  A block that reads a missed expert also waits for the fills'
// victim slots before its fill-through stores (a down block before loading its
// weights).  Waits point only at lower workgroup indices (workgroup 0 first),
// as in the FFN alone.  (A Qwen-like call is 513 workgroups at two per CU: the
// last one starts when another exits, after the victims are out, and stages
// the final plan.)
using ClassifySmall = ClassifySharedT<2048, 2048, 256, 128>;

template <int FMT, int NW, int D, int SPL>
__global__ void __launch_bounds__(NW * WAVE, 4) layer_small_kernel(DecodeParams p, ClassifyParams cp,
                                                                   uint32_t n_gu, uint32_t* sync) {
    __shared__ PlanLds pl;
    constexpr int GU_BYTES = NW * 2 * WAVE * 16;
    constexpr int DN_BYTES = SMALL_H_LDS + NW * WAVE * 16;
    constexpr int CL_BYTES = static_cast<int>(sizeof(ClassifySmall));
    constexpr int RAW = GU_BYTES > DN_BYTES ? (GU_BYTES > CL_BYTES ? GU_BYTES : CL_BYTES)
                                            : (DN_BYTES > CL_BYTES ? DN_BYTES : CL_BYTES);
    __shared__ uint4 raw[(RAW + 15) / 16];
    if (blockIdx.x == 0) {
        classify_body<SPL, NW * WAVE>(cp, *reinterpret_cast<ClassifySmall*>(raw),
                                           sync_word(sync, FL_PLAN), sync_word(sync, FL_VICT));
    } else {
        if (plan_record(cp)) {
            wait_plan_record(sync, blockIdx.x, p, pl);
        } else {
            wait_plan(sync, blockIdx.x, pl, p.err);
            stage_plan_dev(p, pl);
        }
        // with the fills already in the staged plan, the FFN writes them the
        // plain way (gate/up from registers, down stores without a refresh)
        const bool fills = p.has_cache && p.fill_through && !pl.fills_known;
        const uint32_t b = blockIdx.x - 1;
        if (b < n_gu) {
            {   // zero the output for the down blocks' additions
                const int n = p.T * p.H;
                uint32_t* o = reinterpret_cast<uint32_t*>(p.out);
                for (int i = b * (NW * WAVE) + threadIdx.x; i < n; i += n_gu * (NW * WAVE))
                    store_dev(o + i, 0u);
            }
            gate_up_body<FMT, NW, NW, 1, D, true, true>(
                p, pl, *reinterpret_cast<f32x4 (*)[1][NW][1][2][WAVE]>(raw), b, n_gu);
            signal_done(sync, n_gu, b);
            if (fills) copy_gate_up_fills<FMT>(p, pl, sync, b, n_gu);
        } else {
            const int c = b - n_gu;   // two blocks per 16-row tile
            uint32_t old;
            down_rows_body<FMT, NW>(p, pl, raw,
                                    *reinterpret_cast<f32x4 (*)[NW][WAVE]>(raw + SMALL_H_LDS / 16),
                                    (c >> 1) * 16, c & 1, sync, n_gu, fills, old);
            exit_final(sync, old);
            return;
        }
    }
    block_exit(sync);
}

// The fused small-call kernel when the call fits it: at most 16 tokens, gate/up
// items for at most one block per CU, down items for eight wavefronts of
// SMALL_DB each, and h small enough for LDS.
bool small_fits(const DecodeParams& p, int max_uniq) {
    if (p.T > TOK || !(p.H == 1024 || p.H == 2048 || p.H == 4096)) return false;
    if (max_uniq * (p.I / 16) > device_cus() || max_uniq * (p.I / SLAB) > 2 * 8 * SMALL_DB) return false;
    return static_cast<int64_t>(p.T) * p.k * p.I * 4 <= SMALL_H_LDS;
}

template <int FMT>
bool launch_small(const DecodeParams& p, int max_uniq, uint32_t* sync, hipStream_t stream) {
    if (!small_fits(p, max_uniq)) return false;
    const uint32_t n_gu = static_cast<uint32_t>(max_uniq * (p.I / 16));
    const int blocks = static_cast<int>(n_gu) + 2 * (p.H / 16);
    // H / 8 inputs per gate/up wavefront: one or two slabs of each matrix, all
    // in flight at once; four slabs (H = 4096) go through a three-stage ring
    if (p.H <= 2048)
        ffn_small_kernel<FMT, 8, 2><<<blocks, 8 * WAVE, 0, stream>>>(p, n_gu, sync);
    else
        ffn_small_kernel<FMT, 8, 3><<<blocks, 8 * WAVE, 0, stream>>>(p, n_gu, sync);
    return true;
}

template <int FMT>
moe355_status launch_decode(const DecodeParams& p, int max_uniq, uint32_t* sync,
                            hipStream_t stream) {
    moe355_status st;
    const int cus = device_cus();
    if (launch_small<FMT>(p, max_uniq, sync, stream)) return check_launch("expert_ffn_decode");
    if (p.H >= 1024 && p.H <= 4096 && max_uniq * (p.I / 16) <= cus)
        st = launch_gate_up_wide<FMT>(p, max_uniq, stream);
    else if (p.H >= 512)   // wavefronts splitting H: 4 when H >= 512
        st = launch_gate_up<FMT, 4>(p, max_uniq, stream);
    else if (p.H == 256) st = launch_gate_up<FMT, 2>(p, max_uniq, stream);
    else st = launch_gate_up<FMT, 1>(p, max_uniq, stream);
    if (st) return st;
    const int slots = cus * 8;   // eight resident wavefronts per CU
    const int items2 = max_uniq * (p.H / 32);
    const int items1 = max_uniq * (p.H / 16);
    if (items2 >= 2 * slots && p.H % 512 == 0 && 16 * (p.I / 4 + 1) * 16 <= DNL_LDS) {
        // many distinct experts: h in LDS, one block per CU (a window holds a
        // full token group of any expert); four row tiles per wavefront, one
        // slab ahead, sixteen wavefronts (four per SIMD) where H is a multiple
        // of 1024, else eight (DS-like: 154 us per FFN call with sixteen,
        // 156 us with eight, against 168-172 us with two row tiles at any depth
        // and 159-164 us with four tiles 3-6 deep)
        if (p.H % 1024 == 0)
            down_lds_kernel<FMT, 4, 2, 16><<<cus, 16 * WAVE, 0, stream>>>(p);
        else
            down_lds_kernel<FMT, 4, 2, 8><<<cus, 8 * WAVE, 0, stream>>>(p);
    } else if (items2 >= 2 * slots) {
        const int waves = items2 < slots ? items2 : slots;
        down_kernel<FMT, 2, 3, 1, false><<<(waves + 3) / 4, 256, 0, stream>>>(p);
    } else if (items1 <= cus * 4 && p.I >= 256 && p.I <= 1024) {
        // little work: up to four wavefronts per row tile split I (one or two
        // slabs each), all slabs in flight
        if (p.I == 1024) {
            down_kernel<FMT, 1, 3, 4, true><<<items1, 256, 0, stream>>>(p);
        } else if (p.I == 512) {
            down_kernel<FMT, 1, 2, 4, true><<<items1, 256, 0, stream>>>(p);
        } else {
            down_kernel<FMT, 1, 2, 2, true><<<(2 * items1 + 3) / 4, 256, 0, stream>>>(p);
        }
    } else {
        const int waves = items1 < slots ? items1 : slots;
        down_kernel<FMT, 1, 4, 1, false><<<(waves + 3) / 4, 256, 0, stream>>>(p);
    }
    return check_launch("expert_ffn_decode down");
}

__global__ void combine_kernel(int T, int H, int k, const float* __restrict__ y,
                               const float* __restrict__ w, float* __restrict__ out) {
    const int64_t n = static_cast<int64_t>(T) * H;
    for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t t = i / H, c = i - t * H;
        float a = 0.0f;
        for (int j = 0; j < k; ++j) a = fmaf(w[t * k + j], y[(t * k + j) * H + c], a);
        out[i] = a;
    }
}

}  // namespace

size_t decode_ws_bytes(const moe355_layer_desc* d, int T) {
    const size_t tk = static_cast<size_t>(T) * d->top_k;
    return SYNC_BYTES + 2 * tk * d->inter * sizeof(uint16_t);   // h as hi and lo halves
}

namespace {

// Checks a decode FFN call and fills its parameter block.
moe355_status decode_params(const moe355_layer_desc* d, const void* x_bf16, int32_t T,
                            const int32_t* topk_ids, const float* topk_w,
                            const moe355_cache* cache, const uint8_t* pool, int32_t layer,
                            const moe355_classify_out* exp, bool fill_through, float* out,
                            void* ws, size_t ws_bytes, DecodeParams* pp, int* max_uniq_out,
                            uint32_t* err) {
    MOE355_REQUIRE(T >= 0 && T * d->top_k <= 256, MOE355_ENOTSUP,
                   "expert_ffn_decode: T*k=%d outside [0, 256]", T * d->top_k);
    MOE355_REQUIRE(valid_row_len(d->hidden) && valid_row_len(d->inter), MOE355_ENOTSUP,
                   "expert_ffn_decode: H=%d I=%d unsupported", d->hidden, d->inter);
    MOE355_REQUIRE(x_bf16 && topk_ids && topk_w && pool && exp && exp->uniq && exp->counts && out,
                   MOE355_EINVAL, "expert_ffn_decode: null pointer");
    MOE355_REQUIRE(exp->plan && exp->pairs && exp->pair_capacity >= T * d->top_k, MOE355_EINVAL,
                   "expert_ffn_decode: the experts' plan and pairs are required");
    const size_t need = decode_ws_bytes(d, T);
    MOE355_REQUIRE(ws && ws_bytes >= need, MOE355_ECAPACITY,
                   "expert_ffn_decode: workspace %zu < %zu bytes", ws_bytes, need);
    ExpertLayout L;
    expert_layout(d, &L);
    DecodeParams& p = *pp;
    p = DecodeParams{};
    p.x = static_cast<const uint16_t*>(x_bf16);
    p.w = topk_w;
    p.uniq = exp->uniq;
    p.counts = exp->counts;
    p.pool = pool;
    p.S = L.bytes;
    p.E = d->n_experts;
    p.layer = layer;
    p.T = T;
    p.k = d->top_k;
    p.H = d->hidden;
    p.I = d->inter;
    for (int m = 0; m < 3; ++m) {
        p.q_off[m] = L.q_off[m];
        p.s_off[m] = L.s_off[m];
        p.b_off[m] = L.b_off[m];
    }
    const size_t tkI = static_cast<size_t>(T) * d->top_k * d->inter;
    p.h_hi = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + SYNC_BYTES);
    p.h_lo = p.h_hi + tkI;
    p.out = out;
    p.err = err ? err : reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + 256 * SW_ERR);
    if (cache) {
        MOE355_REQUIRE(cache->slot_table && cache->slot_data && cache->slot_bytes == L.bytes &&
                           cache->n_experts == d->n_experts && layer >= 0 &&
                           layer < cache->n_layers,
                       MOE355_EINVAL, "expert_ffn_decode: cache does not match the layer");
        p.has_cache = 1;
        p.slots = cache->slot_data;
        p.fill_through = fill_through ? 1 : 0;
    } else {
        MOE355_REQUIRE(layer >= 0, MOE355_EINVAL, "expert_ffn_decode: layer=%d", layer);
    }
    const int max_uniq = T * d->top_k < d->n_experts ? T * d->top_k : d->n_experts;
    MOE355_REQUIRE(exp->capacity >= max_uniq, MOE355_ECAPACITY,
                   "expert_ffn_decode: plan capacity %d < %d", exp->capacity, max_uniq);
    p.plan = exp->plan;
    p.pairs = exp->pairs;
    p.n_plan = max_uniq;
    *max_uniq_out = max_uniq;
    return ok();
}

template <int FMT>
void launch_layer_small(const DecodeParams& p, const ClassifyParams& cp, int max_uniq,
                        uint32_t* sync, hipStream_t stream) {
    const uint32_t n_gu = static_cast<uint32_t>(max_uniq * (p.I / 16));
    const int blocks = 1 + static_cast<int>(n_gu) + 2 * (p.H / 16);
    // bookkeeping: N / 64 slots per lane in registers for the victim scan
    if (cp.N <= 512) {
        if (p.H <= 2048) layer_small_kernel<FMT, 8, 2, 8><<<blocks, 8 * WAVE, 0, stream>>>(p, cp, n_gu, sync);
        else layer_small_kernel<FMT, 8, 3, 8><<<blocks, 8 * WAVE, 0, stream>>>(p, cp, n_gu, sync);
    } else if (cp.N <= 1024) {
        if (p.H <= 2048) layer_small_kernel<FMT, 8, 2, 16><<<blocks, 8 * WAVE, 0, stream>>>(p, cp, n_gu, sync);
        else layer_small_kernel<FMT, 8, 3, 16><<<blocks, 8 * WAVE, 0, stream>>>(p, cp, n_gu, sync);
    } else {
        if (p.H <= 2048) layer_small_kernel<FMT, 8, 2, 32><<<blocks, 8 * WAVE, 0, stream>>>(p, cp, n_gu, sync);
        else layer_small_kernel<FMT, 8, 3, 32><<<blocks, 8 * WAVE, 0, stream>>>(p, cp, n_gu, sync);
    }
}

}  // namespace

moe355_status decode_layer_small(const moe355_layer_desc* d, const moe355_cache* c,
                                 const uint8_t* pool, int32_t layer, const ClassifyParams& cp,
                                 const void* x_bf16, int32_t T, const int32_t* topk_ids,
                                 const float* topk_w, const moe355_classify_out* lists,
                                 const moe355_evict_policy* pol, float* out, void* ws,
                                 size_t ws_bytes, hipStream_t stream, bool* launched,
                                 uint32_t* err) {
    *launched = false;
    DecodeParams p;
    int max_uniq = 0;
    const moe355_status st = decode_params(d, x_bf16, T, topk_ids, topk_w, c, pool, layer, lists,
                                           true, out, ws, ws_bytes, &p, &max_uniq, err);
    if (st) return st;
    // the bookkeeping workgroup's LDS limits (ClassifySmall) and the FFN's
    if (!small_fits(p, max_uniq) || cp.N > 2048 || cp.E > 256 || T * d->top_k > 128 || pol->K > 128)
        return ok();
    uint32_t* sync = static_cast<uint32_t*>(ws);
    if (d->wfmt == MOE355_W_INT4_G64) launch_layer_small<MOE355_W_INT4_G64>(p, cp, max_uniq, sync, stream);
    else launch_layer_small<MOE355_W_MXFP4>(p, cp, max_uniq, sync, stream);
    *launched = true;
    return check_launch("decode_layer");
}

// Shared by the public decode call and the fused decode-layer call.
moe355_status decode_ffn(const moe355_layer_desc* d, const void* x_bf16, int32_t T,
                         const int32_t* topk_ids, const float* topk_w, const moe355_cache* cache,
                         const uint8_t* pool, int32_t layer, const moe355_classify_out* exp,
                         bool fill_through, float* out, void* ws, size_t ws_bytes,
                         hipStream_t stream, uint32_t* err) {
    if (T == 0) {
        MOE355_REQUIRE(T * d->top_k <= 256 && valid_row_len(d->hidden) && valid_row_len(d->inter),
                       MOE355_ENOTSUP, "expert_ffn_decode: H=%d I=%d unsupported", d->hidden,
                       d->inter);
        return ok();
    }
    DecodeParams p;
    int max_uniq = 0;
    const moe355_status st = decode_params(d, x_bf16, T, topk_ids, topk_w, cache, pool, layer, exp,
                                           fill_through, out, ws, ws_bytes, &p, &max_uniq, err);
    if (st) return st;
    uint32_t* sync = static_cast<uint32_t*>(ws);   // the workspace's first SYNC_BYTES
    if (d->wfmt == MOE355_W_INT4_G64) return launch_decode<MOE355_W_INT4_G64>(p, max_uniq, sync, stream);
    return launch_decode<MOE355_W_MXFP4>(p, max_uniq, sync, stream);
}

}  // namespace moe355

using namespace moe355;

extern "C" moe355_status moe355_expert_ffn_decode(const moe355_layer_desc* d, const void* x_bf16,
                                                  int32_t T, const int32_t* topk_ids,
                                                  const float* topk_w, const moe355_cache* cache,
                                                  const uint8_t* pool, int32_t layer,
                                                  const moe355_classify_out* exp, float* out,
                                                  void* ws, size_t ws_bytes, hipStream_t stream) {
    moe355_status st = check_desc(d);
    if (st) return st;
    return decode_ffn(d, x_bf16, T, topk_ids, topk_w, cache, pool, layer, exp, false, out, ws,
                      ws_bytes, stream);
}

extern "C" moe355_status moe355_combine(int32_t T, int32_t H, int32_t k, const float* y,
                                        const float* topk_w, float* out, hipStream_t stream) {
    MOE355_REQUIRE(T >= 0 && H >= 1 && k >= 1, MOE355_EINVAL, "combine: T=%d H=%d k=%d", T, H, k);
    if (T == 0) return ok();      // an empty batch: nothing to read or write
    MOE355_REQUIRE(y && topk_w && out, MOE355_EINVAL, "combine: null pointer");
    const int64_t n = static_cast<int64_t>(T) * H;
    const int64_t blocks64 = (n + 255) / 256;
    const int blocks = blocks64 < 65536 ? static_cast<int>(blocks64) : 65536;
    combine_kernel<<<blocks, 256, 0, stream>>>(T, H, k, y, topk_w, out);
    return check_launch("combine");
}
