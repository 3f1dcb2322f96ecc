// Decode expert FFN: one kernel per layer call that streams each distinct
// expert's packed weights from HBM once, dequantises them in registers and
// writes the routing-weighted layer output.
//
// [Edge0, section 3.1 "Math contract"]: y = down(silu(gate(x)) * up(x)) per
// routed expert over its quantised weights.  [FT-zh, Core method / Method
// steps]: the GPU computes G = H u F from cache slots while the in-place set is
// read from the pool, the partial sums merge exactly, and the misses chosen for
// filling are batch-copied into their victim slots.
//
// Two launches:
//   gate/up: a work item is (distinct expert, tile of I rows).  Each wavefront
//     owns a fixed 16-byte column chunk of every row (32 weights per lane),
//     keeps its tokens' activations for that chunk in registers and issues all
//     of its row loads first; a block walks a contiguous range of items, so
//     consecutive items share an expert and its converted activations.  int4
//     uses v_dot2_f32_f16 on exact fp16 nibbles (1024 + q with 1024 removed in
//     packed fp16) against fp16 activations and applies s * sum(q x) +
//     b * sum(x) per 64-group; MXFP4 converts codes with the gfx950 scaled
//     fp4 -> fp16 conversion and scales each 32-block by 2^(e-127).
//     h = silu(g) * u goes to the workspace in fp32.  This launch also zeroes the
//     layer output.
//   down + combine: a work item is (distinct expert, tile of H rows).  The
//     expert's h slices are loaded once per item and reused across its rows;
//     each row's dot product meets the routing weight and is added into the
//     layer output with an fp32 atomic (k additions per output element).
//
// Before anything else every block stages the call's plan (for each distinct
// expert: where its bytes live, whether this call fills a cache slot with it,
// and its routed pairs) in LDS, so every weight load is independent of the
// others.  With fill-through on, an expert that this call fills into a cache
// slot is read from the pool and its bytes are written to the slot by the lanes
// that read them, which replaces the separate pool -> slot copy.
#include <stdlib.h>

#include "internal.h"

namespace moe355 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

struct DecodeParams {
    const uint16_t* x;
    const int32_t* ids;
    const float* w;
    const int32_t* uniq;
    const int32_t* counts;
    const int32_t* table;
    const uint8_t* slots;
    const uint8_t* pool;
    const int32_t* plan;     // [n_plan][4]: slot or -1, filled now, first pair, pair count
    const int32_t* pairs;    // routed pairs grouped by expert
    int n_plan;              // plan rows loaded (>= number of distinct experts)
    int fill_through;
    int64_t S;
    int E, layer, T, k, H, I;
    int64_t q_off[3], s_off[3], b_off[3];
    float* h;
    float* out;
};

struct ExpertRef {
    const uint8_t* src;
    uint8_t* dst;  // fill-through destination slot, or null
};

// The per-call plan, staged in LDS by every block before any weight load.
constexpr int MAX_PLAN = 256;
struct PlanLds {
    int4 plan[MAX_PLAN];
    int32_t uniq[MAX_PLAN];
    int32_t pairs[MAX_PLAN];
    int32_t n_uniq;
};

// Where distinct expert u's bytes are read from (and written to, with fill-through).
__device__ __forceinline__ ExpertRef expert_ref(const DecodeParams& p, const PlanLds& pl, int u) {
    const int4 row = pl.plan[u];
    const uint8_t* from_pool = p.pool + (static_cast<int64_t>(p.layer) * p.E + pl.uniq[u]) * p.S;
    ExpertRef r;
    r.dst = nullptr;
    r.src = from_pool;
    if (p.table && row.x >= 0) {
        uint8_t* slot = const_cast<uint8_t*>(p.slots) + static_cast<int64_t>(row.x) * p.S;
        if (p.fill_through && row.y) {
            r.dst = slot;        // filled by this call: read the pool, write the slot
        } else {
            r.src = slot;
        }
    }
    return r;
}

// Every block stages the plan first: one round trip, then loads are independent.
__device__ __forceinline__ void stage_plan(const DecodeParams& p, PlanLds& pl) {
    if (threadIdx.x < p.n_plan) {
        pl.plan[threadIdx.x] = reinterpret_cast<const int4*>(p.plan)[threadIdx.x];
        pl.uniq[threadIdx.x] = p.uniq[threadIdx.x];
    }
    if (threadIdx.x < p.T * p.k) pl.pairs[threadIdx.x] = p.pairs[threadIdx.x];
    if (threadIdx.x == 0) pl.n_uniq = p.counts[0];
    __syncthreads();
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
    return e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
}

__device__ __forceinline__ half2_t as_half2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

__device__ __forceinline__ uint4 ldg16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

// The 32 bf16 activations under one 16-byte weight chunk as fp16 pairs, paired
// the way the chunk's codes unpack; returns their fp32 sum.
template <int FMT>
__device__ __forceinline__ float load_x_pairs(const uint16_t* xs, half2_t xh[16]) {
    const uint4* v = reinterpret_cast<const uint4*>(xs);
    float xf[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 q = v[i];
        const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            xf[8 * i + 2 * j] = __uint_as_float(d[j] << 16);
            xf[8 * i + 2 * j + 1] = __uint_as_float(d[j] & 0xFFFF0000u);
        }
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) sum += xf[i];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        // int4: dword d unpacks to pairs (8d+s, 8d+4+s); MXFP4: natural pairs
        const int a = FMT == MOE355_W_INT4_G64 ? 8 * (i / 4) + (i % 4) : 2 * i;
        const int b = FMT == MOE355_W_INT4_G64 ? a + 4 : a + 1;
        half2_t t;
        t.x = static_cast<_Float16>(xf[a]);
        t.y = static_cast<_Float16>(xf[b]);
        xh[i] = t;
    }
    return sum;
}

// Exact fp16 nibbles of one int4 chunk, pairs (8d+s, 8d+4+s).
__device__ __forceinline__ void unpack_int4_f16(uint4 w, half2_t q[16]) {
    const uint32_t d4[4] = {w.x, w.y, w.z, w.w};
    const half2_t k1024 = {static_cast<_Float16>(1024.0f), static_cast<_Float16>(1024.0f)};
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            q[4 * d + s] = as_half2(((d4[d] >> (4 * s)) & 0x000F000Fu) | 0x64006400u) - k1024;
}

// fp16 e2m1 values of one MXFP4 chunk, natural pairs (2i, 2i+1).
__device__ __forceinline__ void unpack_fp4_f16(uint4 w, half2_t q[16]) {
    const uint32_t d4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        q[4 * d + 0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d4[d], 1.0f, 0);
        q[4 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d4[d], 1.0f, 1);
        q[4 * d + 2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d4[d], 1.0f, 2);
        q[4 * d + 3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d4[d], 1.0f, 3);
    }
}

__device__ __forceinline__ float dot16(const half2_t q[16], const half2_t x[16]) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = __builtin_amdgcn_fdot2(q[i], x[i], a, false);
    return a;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// One row chunk of a matrix: packed codes plus its scale (and bias for int4).
struct Chunk {
    uint4 q;
    uint32_t s, b;
};

// Load (and with fill-through, copy) the chunk `ch` (16 bytes) of row r of matrix m.
template <int FMT>
__device__ __forceinline__ Chunk load_chunk(const DecodeParams& p, const ExpertRef& ref, int m,
                                            int64_t row_bytes, int L, int r, int ch) {
    Chunk c;
    const int64_t qo = p.q_off[m] + r * row_bytes + ch * 16;
    c.q = ldg16(ref.src + qo);
    if (FMT == MOE355_W_INT4_G64) {
        const int64_t g = static_cast<int64_t>(r) * (L / 64) + ch / 2;
        c.s = reinterpret_cast<const uint16_t*>(ref.src + p.s_off[m])[g];
        c.b = reinterpret_cast<const uint16_t*>(ref.src + p.b_off[m])[g];
        if (ref.dst) {
            *reinterpret_cast<uint4*>(ref.dst + qo) = c.q;
            if ((ch & 1) == 0) {
                reinterpret_cast<uint16_t*>(ref.dst + p.s_off[m])[g] = static_cast<uint16_t>(c.s);
                reinterpret_cast<uint16_t*>(ref.dst + p.b_off[m])[g] = static_cast<uint16_t>(c.b);
            }
        }
    } else {
        const int64_t eo = p.s_off[m] + static_cast<int64_t>(r) * (L / 32) + ch;
        c.s = ref.src[eo];
        c.b = 0;
        if (ref.dst) {
            *reinterpret_cast<uint4*>(ref.dst + qo) = c.q;
            ref.dst[eo] = static_cast<uint8_t>(c.s);
        }
    }
    return c;
}

// Convert one pair group's activations (one or two tokens) for this lane's chunks.
template <int FMT, int NC>
__device__ __forceinline__ void load_group_x(const DecodeParams& p, int t0, int t1, int ch0,
                                             half2_t xh[2][NC][16], float xs[2][NC]) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int64_t col = static_cast<int64_t>(ch0 + c * WAVE) * 32;
        xs[0][c] = load_x_pairs<FMT>(p.x + static_cast<int64_t>(t0) * p.H + col, xh[0][c]);
        if (t1 >= 0) xs[1][c] = load_x_pairs<FMT>(p.x + static_cast<int64_t>(t1) * p.H + col, xh[1][c]);
    }
}

// gate . x and up . x for one row (LA loads of it) and one or two tokens.
template <int FMT, int NC, int LA>
__device__ __forceinline__ void gate_up_rows(const DecodeParams& p, const Chunk wc[2][LA][NC],
                                             const half2_t xh[2][NC][16], const float xs[2][NC],
                                             bool two, int seg, int ch0, int r0, int rpw,
                                             int pr0, int pr1) {
#pragma unroll
    for (int l = 0; l < LA; ++l) {
        float acc[2][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                half2_t q[16];
                float s, b;
                if (FMT == MOE355_W_INT4_G64) {
                    unpack_int4_f16(wc[m][l][c].q, q);
                    s = bf16_to_f32(static_cast<uint16_t>(wc[m][l][c].s));
                    b = bf16_to_f32(static_cast<uint16_t>(wc[m][l][c].b));
                } else {
                    unpack_fp4_f16(wc[m][l][c].q, q);
                    s = e8m0_to_f32(wc[m][l][c].s);
                    b = 0.0f;
                }
                const float d0 = dot16(q, xh[0][c]);
                acc[m][0] += FMT == MOE355_W_INT4_G64 ? fmaf(s, d0, b * xs[0][c]) : s * d0;
                if (two) {
                    const float d1 = dot16(q, xh[1][c]);
                    acc[m][1] += FMT == MOE355_W_INT4_G64 ? fmaf(s, d1, b * xs[1][c]) : s * d1;
                }
            }
            acc[m][0] = segment_sum_f32(acc[m][0], seg);
            if (two) acc[m][1] = segment_sum_f32(acc[m][1], seg);
        }
        if (ch0 == 0) {
            const int r = r0 + l * rpw;
            p.h[static_cast<int64_t>(pr0) * p.I + r] = silu(acc[0][0]) * acc[1][0];
            if (two) p.h[static_cast<int64_t>(pr1) * p.I + r] = silu(acc[0][1]) * acc[1][1];
        }
    }
}

// NC: 16-byte chunks per lane per row (H / 2048, or 1 for rows narrower than a
// wavefront); LA: row loads per wavefront per work item.
template <int FMT, int NC, int LA>
__global__ void __launch_bounds__(256) gate_up_kernel(DecodeParams p, int seg) {
    __shared__ PlanLds pl;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wv = threadIdx.x / WAVE;
    stage_plan(p, pl);
    {   // zero the layer output for the down launch's atomics
        const int64_t n = static_cast<int64_t>(p.T) * p.H;
        for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
             i += static_cast<int64_t>(gridDim.x) * blockDim.x)
            p.out[i] = 0.0f;
    }
    const int rpw = WAVE / seg;
    const int wave_rows = LA * rpw;
    const int item_rows = 4 * wave_rows;
    const int tiles = p.I / item_rows;
    const int n_items = pl.n_uniq * tiles;
    const int per = (n_items + gridDim.x - 1) / gridDim.x;
    const int sub = lane / seg, ch0 = lane % seg;
    const int64_t row_bytes = p.H / 2;
    half2_t xh[2][NC][16];
    float xs[2][NC];
    int cached_u = -1;   // expert whose first pair group sits in xh / xs
    const int i_end = min(n_items, (static_cast<int>(blockIdx.x) + 1) * per);
    for (int item = blockIdx.x * per; item < i_end; ++item) {
        const int u = item / tiles;
        const int tile = item - u * tiles;
        const int r0 = tile * item_rows + wv * wave_rows + sub;
        const ExpertRef ref = expert_ref(p, pl, u);
        Chunk wc[2][LA][NC];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int l = 0; l < LA; ++l)
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    wc[m][l][c] = load_chunk<FMT>(p, ref, m, row_bytes, p.H, r0 + l * rpw,
                                                  ch0 + c * WAVE);
        const int pb = pl.plan[u].z, pc = pl.plan[u].w;
        for (int g = 0; g < pc; g += 2) {
            const int pr0 = pl.pairs[pb + g];
            const int pr1 = g + 1 < pc ? pl.pairs[pb + g + 1] : -1;
            if (g > 0 || cached_u != u) {
                load_group_x<FMT, NC>(p, pr0 / p.k, pr1 >= 0 ? pr1 / p.k : -1, ch0, xh, xs);
                cached_u = g == 0 ? u : -1;
            }
            if (pr1 >= 0)
                gate_up_rows<FMT, NC, LA>(p, wc, xh, xs, true, seg, ch0, r0, rpw, pr0, pr1);
            else
                gate_up_rows<FMT, NC, LA>(p, wc, xh, xs, false, seg, ch0, r0, rpw, pr0, -1);
        }
    }
}

// One pair's h slice for this lane's chunks, with its fp32 sum.
template <int NC>
__device__ __forceinline__ void load_h(const DecodeParams& p, int pr, int ch0, float hv[NC][32],
                                       float hs[NC]) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const float4* hp = reinterpret_cast<const float4*>(
            p.h + static_cast<int64_t>(pr) * p.I + (ch0 + c * WAVE) * 32);
        hs[c] = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 v = hp[i];
            hv[c][4 * i + 0] = v.x;
            hv[c][4 * i + 1] = v.y;
            hv[c][4 * i + 2] = v.z;
            hv[c][4 * i + 3] = v.w;
            hs[c] += (v.x + v.y) + (v.z + v.w);
        }
    }
}

// down_row . h for one 16-byte chunk (32 weights) against this lane's h slice.
template <int FMT>
__device__ __forceinline__ float down_chunk_dot(const Chunk& ch, const float hv[32], float hs) {
    const uint32_t d4[4] = {ch.q.x, ch.q.y, ch.q.z, ch.q.w};
    float dq = 0.0f;
    if (FMT == MOE355_W_INT4_G64) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t lo = d4[d] & 0x0F0F0F0Fu;
            const uint32_t hi = (d4[d] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                dq = fmaf(static_cast<float>((lo >> (8 * b)) & 0xFFu), hv[8 * d + 2 * b], dq);
                dq = fmaf(static_cast<float>((hi >> (8 * b)) & 0xFFu), hv[8 * d + 2 * b + 1], dq);
            }
        }
        return fmaf(bf16_to_f32(static_cast<uint16_t>(ch.s)), dq,
                    bf16_to_f32(static_cast<uint16_t>(ch.b)) * hs);
    } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const float2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d4[d], 1.0f, 0);
            const float2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d4[d], 1.0f, 1);
            const float2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d4[d], 1.0f, 2);
            const float2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d4[d], 1.0f, 3);
            dq = fmaf(v0.x, hv[8 * d + 0], dq);
            dq = fmaf(v0.y, hv[8 * d + 1], dq);
            dq = fmaf(v1.x, hv[8 * d + 2], dq);
            dq = fmaf(v1.y, hv[8 * d + 3], dq);
            dq = fmaf(v2.x, hv[8 * d + 4], dq);
            dq = fmaf(v2.y, hv[8 * d + 5], dq);
            dq = fmaf(v3.x, hv[8 * d + 6], dq);
            dq = fmaf(v3.y, hv[8 * d + 7], dq);
        }
        return e8m0_to_f32(ch.s) * dq;
    }
}

// Down rows [r0 + l*rpw] for one or two pairs whose h slices are in registers.
template <int FMT, int NC, int LC>
__device__ __forceinline__ void down_rows(const DecodeParams& p, const Chunk wc[LC][NC],
                                          const float hv[2][NC][32], const float hs[2][NC],
                                          bool two, int seg, int ch0, int r0, int rpw, float* o0,
                                          float w0, float* o1, float w1) {
#pragma unroll
    for (int l = 0; l < LC; ++l) {
        float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            a0 += down_chunk_dot<FMT>(wc[l][c], hv[0][c], hs[0][c]);
            if (two) a1 += down_chunk_dot<FMT>(wc[l][c], hv[1][c], hs[1][c]);
        }
        a0 = segment_sum_f32(a0, seg);
        if (two) a1 = segment_sum_f32(a1, seg);
        if (ch0 == 0) {
            unsafeAtomicAdd(o0 + r0 + l * rpw, w0 * a0);
            if (two) unsafeAtomicAdd(o1 + r0 + l * rpw, w1 * a1);
        }
    }
}

// A work item is (distinct expert, tile of H rows); each wavefront streams nch
// chunks of LC row loads, prefetching the next chunk while it computes one, with
// the h slices of up to two routed pairs held in registers for the whole item.
template <int FMT, int NC, int LC>
__global__ void __launch_bounds__(256) down_kernel(DecodeParams p, int seg, int nch) {
    __shared__ PlanLds pl;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wv = threadIdx.x / WAVE;
    stage_plan(p, pl);
    const int rpw = WAVE / seg;
    const int wave_rows = LC * nch * rpw;
    const int item_rows = 4 * wave_rows;
    const int tiles = p.H / item_rows;
    const int n_items = pl.n_uniq * tiles;
    const int per = (n_items + gridDim.x - 1) / gridDim.x;
    const int sub = lane / seg, ch0 = lane % seg;
    const int64_t row_bytes = p.I / 2;
    const int i_end = min(n_items, (static_cast<int>(blockIdx.x) + 1) * per);
    for (int item = blockIdx.x * per; item < i_end; ++item) {
        const int u = item / tiles;
        const int tile = item - u * tiles;
        const int rbase = tile * item_rows + wv * wave_rows + sub;
        const ExpertRef ref = expert_ref(p, pl, u);
        const int pb = pl.plan[u].z, pc = pl.plan[u].w;
        for (int g = 0; g < pc; g += 2) {
            const int pr0 = pl.pairs[pb + g];
            const int pr1 = g + 1 < pc ? pl.pairs[pb + g + 1] : -1;
            const bool two = pr1 >= 0;
            float hv[2][NC][32], hs[2][NC];
            load_h<NC>(p, pr0, ch0, hv[0], hs[0]);
            if (two) load_h<NC>(p, pr1, ch0, hv[1], hs[1]);
            float* o0 = p.out + static_cast<int64_t>(pr0 / p.k) * p.H;
            float* o1 = two ? p.out + static_cast<int64_t>(pr1 / p.k) * p.H : o0;
            const float w0 = p.w[pr0], w1 = two ? p.w[pr1] : 0.0f;
            // only the first pair group copies the bytes into a filled slot
            ExpertRef rf = ref;
            if (g > 0) rf.dst = nullptr;
            Chunk cur[LC][NC], nxt[LC][NC];
#pragma unroll
            for (int l = 0; l < LC; ++l)
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    cur[l][c] = load_chunk<FMT>(p, rf, 2, row_bytes, p.I, rbase + l * rpw,
                                                ch0 + c * WAVE);
#pragma unroll 1
            for (int ci = 0; ci < nch; ++ci) {
                const int r0 = rbase + ci * LC * rpw;
                if (ci + 1 < nch) {
#pragma unroll
                    for (int l = 0; l < LC; ++l)
#pragma unroll
                        for (int c = 0; c < NC; ++c)
                            nxt[l][c] = load_chunk<FMT>(p, rf, 2, row_bytes, p.I,
                                                        r0 + (LC + l) * rpw, ch0 + c * WAVE);
                }
                if (two)
                    down_rows<FMT, NC, LC>(p, cur, hv, hs, true, seg, ch0, r0, rpw, o0, w0, o1, w1);
                else
                    down_rows<FMT, NC, LC>(p, cur, hv, hs, false, seg, ch0, r0, rpw, o0, w0, o1, w1);
                if (ci + 1 < nch) {
#pragma unroll
                    for (int l = 0; l < LC; ++l)
#pragma unroll
                        for (int c = 0; c < NC; ++c) cur[l][c] = nxt[l][c];
                }
            }
        }
    }
}

// Row geometry: lanes per row segment and 16-byte chunks per lane for rows of L weights.
void row_geometry(int L, int* seg, int* nc) {
    const int chunks = L / 32;
    if (chunks >= WAVE) {
        *seg = WAVE;
        *nc = chunks / WAVE;
    } else {
        *seg = chunks;
        *nc = 1;
    }
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

template <int FMT, int NCA, int LA, int NCB, int LC>
moe355_status launch_two(const DecodeParams& p, int segA, int segB, int max_uniq,
                         hipStream_t stream) {
    const int rpw_b = WAVE / segB;
    const int rows_a = 4 * LA * (WAVE / segA);
    MOE355_REQUIRE(p.I % rows_a == 0 && p.H % (4 * LC * rpw_b) == 0, MOE355_ENOTSUP,
                   "expert_ffn_decode: H=%d I=%d do not tile", p.H, p.I);
    const int cap = device_cus() * 2;        // two resident blocks per CU
    // down: as many row chunks per item as keep at least two items per CU (reuse
    // of the h slices grows with the chunks), at most 8
    const int base_tiles = p.H / (4 * LC * rpw_b);
    int nch = 8;
    while (nch > 1 && (base_tiles % nch != 0 || max_uniq * (base_tiles / nch) < 2 * device_cus()))
        nch >>= 1;
    const int items_a = max_uniq * (p.I / rows_a);
    const int items_b = max_uniq * (base_tiles / nch);
    gate_up_kernel<FMT, NCA, LA><<<items_a < cap ? items_a : cap, 256, 0, stream>>>(p, segA);
    moe355_status st = check_launch("expert_ffn_decode gate_up");
    if (st) return st;
    down_kernel<FMT, NCB, LC><<<items_b < cap ? items_b : cap, 256, 0, stream>>>(p, segB, nch);
    return check_launch("expert_ffn_decode down");
}

template <int FMT>
moe355_status launch_decode(const DecodeParams& p, int max_uniq, hipStream_t stream) {
    int segA, ncA, segB, ncB;
    row_geometry(p.H, &segA, &ncA);
    row_geometry(p.I, &segB, &ncB);
    // gate/up: 4 row loads per wavefront and item (2 with two chunks per row);
    // down: chunks of 4 row loads per wavefront (2 with two chunks per row)
    if (ncA == 1 && ncB == 1) return launch_two<FMT, 1, 4, 1, 4>(p, segA, segB, max_uniq, stream);
    if (ncA == 2 && ncB == 1) return launch_two<FMT, 2, 2, 1, 4>(p, segA, segB, max_uniq, stream);
    if (ncA == 2 && ncB == 2) return launch_two<FMT, 2, 2, 2, 2>(p, segA, segB, max_uniq, stream);
    if (ncA == 1 && ncB == 2) return launch_two<FMT, 1, 4, 2, 2>(p, segA, segB, max_uniq, stream);
    return fail(MOE355_ENOTSUP, "expert_ffn_decode: H=%d I=%d", p.H, p.I);
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
    return 256 + tk * d->inter * sizeof(float);
}

// Shared by the public decode call and the fused decode-layer call.
moe355_status decode_ffn(const moe355_layer_desc* d, const void* x_bf16, int32_t T,
                         const int32_t* topk_ids, const float* topk_w, const moe355_cache* cache,
                         const uint8_t* pool, int32_t layer, const moe355_classify_out* exp,
                         bool fill_through, float* out, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
    MOE355_REQUIRE(T >= 0 && T * d->top_k <= 256, MOE355_ENOTSUP,
                   "expert_ffn_decode: T*k=%d outside [0, 256]", T * d->top_k);
    MOE355_REQUIRE(valid_row_len(d->hidden) && valid_row_len(d->inter), MOE355_ENOTSUP,
                   "expert_ffn_decode: H=%d I=%d unsupported", d->hidden, d->inter);
    if (T == 0) return ok();
    MOE355_REQUIRE(x_bf16 && topk_ids && topk_w && pool && exp && exp->uniq && exp->counts && out,
                   MOE355_EINVAL, "expert_ffn_decode: null pointer");
    MOE355_REQUIRE(exp->plan && exp->pairs && exp->pair_capacity >= T * d->top_k, MOE355_EINVAL,
                   "expert_ffn_decode: the experts' plan and pairs are required");
    const size_t need = decode_ws_bytes(d, T);
    MOE355_REQUIRE(ws && ws_bytes >= need, MOE355_ECAPACITY,
                   "expert_ffn_decode: workspace %zu < %zu bytes", ws_bytes, need);
    ExpertLayout L;
    expert_layout(d, &L);
    DecodeParams p{};
    p.x = static_cast<const uint16_t*>(x_bf16);
    p.ids = topk_ids;
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
    p.h = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + 256);
    p.out = out;
    if (cache) {
        MOE355_REQUIRE(cache->slot_table && cache->slot_data && cache->slot_bytes == L.bytes &&
                           cache->n_experts == d->n_experts && layer >= 0 &&
                           layer < cache->n_layers,
                       MOE355_EINVAL, "expert_ffn_decode: cache does not match the layer");
        p.table = cache->slot_table;
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
    if (d->wfmt == MOE355_W_INT4_G64) return launch_decode<MOE355_W_INT4_G64>(p, max_uniq, stream);
    return launch_decode<MOE355_W_MXFP4>(p, max_uniq, stream);
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
    MOE355_REQUIRE(y && topk_w && out, MOE355_EINVAL, "combine: null pointer");
    if (T == 0) return ok();
    const int64_t n = static_cast<int64_t>(T) * H;
    const int64_t blocks64 = (n + 255) / 256;
    const int blocks = blocks64 < 65536 ? static_cast<int>(blocks64) : 65536;
    combine_kernel<<<blocks, 256, 0, stream>>>(T, H, k, y, topk_w, out);
    return check_launch("combine");
}
