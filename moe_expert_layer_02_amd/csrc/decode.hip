// Decode expert FFN: a grouped GEMV that streams each distinct expert's packed
// weights from HBM once and dequantises them in registers, with the weighted
// combine fused into the down projection.
//
// [Edge0, section 3.1 "Math contract"]: y = down(silu(gate(x)) * up(x)) per
// routed expert over its quantised weights.  [FT-zh, Core method]: the GPU
// computes G = H u F from cache slots, the in-place set comes from the pool, and
// partial sums merge exactly; here both read paths feed the same kernel.
//
// Layout of work:
//   gate_up kernel: a work item is (distinct expert, tile of I rows); each
//     wavefront owns a fixed column slice of every row (16 bytes = 32 weights
//     per lane per load), keeps its tokens' activations for that slice in
//     registers and issues all of its row loads before computing.  int4 gate/up
//     use v_dot2_f32_f16 on exact fp16 nibbles (1024 + q with the 1024 removed
//     in packed fp16) against fp16 activations; per 64-group the partial is
//     s * sum(q x) + b * sum(x).  MXFP4 converts codes with the gfx950 scaled
//     fp4 -> fp16 conversion and applies 2^(e-127) per 32-block in fp32.
//     h = silu(g) * u is written once per (token, row) in fp32.
//   down kernel: a work item is a tile of H rows for *all* distinct experts of
//     the call; it accumulates sum_j w_j y_j per (token, row) in LDS in a fixed
//     expert order and writes the layer output once: no atomics, no zero fill,
//     run-to-run identical.  h stays fp32; weights become fp32 and meet it in
//     fp32 FMAs.
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
    int64_t S;
    int E, layer, T, k, H, I;
    int64_t q_off[3], s_off[3], b_off[3];
    float* h;
    float* out;
};

__device__ __forceinline__ const uint8_t* expert_ptr(const DecodeParams& p, int e) {
    if (p.table) {
        const int s = p.table[p.layer * p.E + e];
        if (s >= 0) return p.slots + static_cast<int64_t>(s) * p.S;
    }
    return p.pool + (static_cast<int64_t>(p.layer) * p.E + e) * p.S;
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
    return e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
}

__device__ __forceinline__ half2_t as_half2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

__device__ __forceinline__ uint4 ldg16(const uint8_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}

// Ballot masks of the pairs (t*k + j) routed to expert e (T*k <= 256).
__device__ __forceinline__ void pair_masks(const DecodeParams& p, int e, int lane, uint64_t m[4]) {
    const int n = p.T * p.k;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int idx = c * WAVE + lane;
        const bool hit = idx < n && p.ids[idx] == e;
        m[c] = __ballot(hit);
    }
}

// Pop the next routed pair from the masks (wave-uniform); -1 when none is left.
__device__ __forceinline__ int next_pair(uint64_t m[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if (m[c]) {
            const int b = __ffsll(static_cast<long long>(m[c])) - 1;
            m[c] &= m[c] - 1;
            return c * WAVE + b;
        }
    }
    return -1;
}

// The 32 bf16 activations of one 16-byte weight chunk as fp16 pairs, paired the
// way the chunk's nibbles unpack.  Returns their fp32 sum.
template <int FMT>
__device__ __forceinline__ float load_x_pairs(const uint16_t* xs, half2_t xh[16]) {
    const uint4* v = reinterpret_cast<const uint4*>(xs);
    uint32_t wds[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint4 q = v[i];
        wds[4 * i + 0] = q.x;
        wds[4 * i + 1] = q.y;
        wds[4 * i + 2] = q.z;
        wds[4 * i + 3] = q.w;
    }
    float xf[32];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        xf[2 * i] = __uint_as_float(wds[i] << 16);
        xf[2 * i + 1] = __uint_as_float(wds[i] & 0xFFFF0000u);
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) sum += xf[i];
    if (FMT == MOE355_W_INT4_G64) {
        // dword d of the chunk unpacks to pairs (8d+s, 8d+4+s), s = 0..3
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                half2_t t;
                t.x = static_cast<_Float16>(xf[8 * d + s]);
                t.y = static_cast<_Float16>(xf[8 * d + 4 + s]);
                xh[4 * d + s] = t;
            }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            half2_t t;
            t.x = static_cast<_Float16>(xf[2 * i]);
            t.y = static_cast<_Float16>(xf[2 * i + 1]);
            xh[i] = t;
        }
    }
    return sum;
}

// Exact fp16 nibbles of one 16-byte int4 chunk, pairs (8d+s, 8d+4+s).
__device__ __forceinline__ void unpack_int4_f16(uint4 w, half2_t q[16]) {
    const uint32_t d4[4] = {w.x, w.y, w.z, w.w};
    const half2_t k1024 = {static_cast<_Float16>(1024.0f), static_cast<_Float16>(1024.0f)};
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            q[4 * d + s] = as_half2(((d4[d] >> (4 * s)) & 0x000F000Fu) | 0x64006400u) - k1024;
}

// fp16 e2m1 values of one 16-byte MXFP4 chunk, natural pairs (2i, 2i+1).
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

// ---------------------------------------------------------------------------
// gate / up:  h[pair, r] = silu(gate_r . x_t) * (up_r . x_t)
// NC: 16-byte chunks per lane per row (H / 2048, or 1 when a row is narrower
// than a wavefront); LOADS: row loads per wavefront per work item; TG: tokens
// whose activations are held in registers at once.
template <int FMT, int NC, int LOADS, int TG>
__global__ void __launch_bounds__(256) gate_up_kernel(DecodeParams p, int seg) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int wv = threadIdx.x / WAVE;
    const int rpw = WAVE / seg;            // rows per wavefront load
    const int sub = lane / seg;            // row of this lane within a load
    const int ch0 = lane % seg;            // first 16-byte chunk of this lane
    const int wave_rows = LOADS * rpw;
    const int item_rows = 4 * wave_rows;
    const int tiles = p.I / item_rows;
    const int n_items = p.counts[0] * tiles;
    const int64_t row_bytes = p.H / 2;

    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int u = item / tiles;
        const int tile = item - u * tiles;
        const int e = p.uniq[u];
        const uint8_t* base = expert_ptr(p, e);
        const int r0 = tile * item_rows + wv * wave_rows + sub;

        // issue every weight load of this wavefront first
        uint4 wgt[2][LOADS][NC];
        uint32_t sc[2][LOADS][NC], bi[2][LOADS][NC];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int l = 0; l < LOADS; ++l) {
                const int r = r0 + l * rpw;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int ch = ch0 + c * WAVE;
                    wgt[m][l][c] = ldg16(base + p.q_off[m] + r * row_bytes + ch * 16);
                    if (FMT == MOE355_W_INT4_G64) {
                        const int64_t g = static_cast<int64_t>(r) * (p.H / 64) + ch / 2;
                        sc[m][l][c] = reinterpret_cast<const uint16_t*>(base + p.s_off[m])[g];
                        bi[m][l][c] = reinterpret_cast<const uint16_t*>(base + p.b_off[m])[g];
                    } else {
                        sc[m][l][c] = base[p.s_off[m] + static_cast<int64_t>(r) * (p.H / 32) + ch];
                        bi[m][l][c] = 0;
                    }
                }
            }

        uint64_t masks[4];
        pair_masks(p, e, lane, masks);
        for (;;) {
            int pr[TG];
            int np = 0;
#pragma unroll
            for (int i = 0; i < TG; ++i) {
                pr[i] = next_pair(masks);
                np += pr[i] >= 0 ? 1 : 0;
            }
            if (np == 0) break;
            half2_t xh[TG][NC][16];
            float xs[TG][NC];
#pragma unroll
            for (int i = 0; i < TG; ++i)
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    if (pr[i] >= 0) {
                        const int t = pr[i] / p.k;
                        const int ch = ch0 + c * WAVE;
                        xs[i][c] = load_x_pairs<FMT>(p.x + static_cast<int64_t>(t) * p.H + ch * 32,
                                                     xh[i][c]);
                    } else {
                        xs[i][c] = 0.0f;
#pragma unroll
                        for (int j = 0; j < 16; ++j) xh[i][c][j] = half2_t{0, 0};
                    }
                }
#pragma unroll
            for (int l = 0; l < LOADS; ++l) {
                float acc[2][TG];
#pragma unroll
                for (int m = 0; m < 2; ++m) {
#pragma unroll
                    for (int i = 0; i < TG; ++i) acc[m][i] = 0.0f;
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        half2_t q[16];
                        float s, b;
                        if (FMT == MOE355_W_INT4_G64) {
                            unpack_int4_f16(wgt[m][l][c], q);
                            s = bf16_to_f32(static_cast<uint16_t>(sc[m][l][c]));
                            b = bf16_to_f32(static_cast<uint16_t>(bi[m][l][c]));
                        } else {
                            unpack_fp4_f16(wgt[m][l][c], q);
                            s = e8m0_to_f32(sc[m][l][c]);
                            b = 0.0f;
                        }
#pragma unroll
                        for (int i = 0; i < TG; ++i) {
                            const float d = dot16(q, xh[i][c]);
                            acc[m][i] += FMT == MOE355_W_INT4_G64 ? fmaf(s, d, b * xs[i][c]) : s * d;
                        }
                    }
#pragma unroll
                    for (int i = 0; i < TG; ++i) acc[m][i] = segment_sum_f32(acc[m][i], seg);
                }
                if (ch0 == 0) {
                    const int r = r0 + l * rpw;
#pragma unroll
                    for (int i = 0; i < TG; ++i)
                        if (pr[i] >= 0)
                            p.h[static_cast<int64_t>(pr[i]) * p.I + r] = silu(acc[0][i]) * acc[1][i];
                }
            }
            if (np < TG) break;
        }
    }
}

// ---------------------------------------------------------------------------
// down + combine: out[t, n] = sum over the call's experts e and pairs (t, j)
// routed to e of w[t, j] * (down_e[n, :] . h[t*k + j, :]).
template <int FMT, int NC, int LOADS>
__global__ void __launch_bounds__(256) down_kernel(DecodeParams p, int seg) {
    extern __shared__ float acc_lds[];  // [T][item_rows]
    const int lane = threadIdx.x & (WAVE - 1);
    const int wv = threadIdx.x / WAVE;
    const int rpw = WAVE / seg;
    const int sub = lane / seg;
    const int ch0 = lane % seg;
    const int wave_rows = LOADS * rpw;
    const int item_rows = 4 * wave_rows;
    const int n_items = p.H / item_rows;
    const int n_uniq = p.counts[0];
    const int64_t row_bytes = p.I / 2;

    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        for (int i = threadIdx.x; i < p.T * item_rows; i += blockDim.x) acc_lds[i] = 0.0f;
        __syncthreads();
        const int rl0 = wv * wave_rows + sub;          // local row of load 0
        const int r0 = item * item_rows + rl0;
        for (int u = 0; u < n_uniq; ++u) {
            const int e = p.uniq[u];
            const uint8_t* base = expert_ptr(p, e);
            uint4 wgt[LOADS][NC];
            uint32_t sc[LOADS][NC], bi[LOADS][NC];
#pragma unroll
            for (int l = 0; l < LOADS; ++l) {
                const int r = r0 + l * rpw;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int ch = ch0 + c * WAVE;
                    wgt[l][c] = ldg16(base + p.q_off[2] + r * row_bytes + ch * 16);
                    if (FMT == MOE355_W_INT4_G64) {
                        const int64_t g = static_cast<int64_t>(r) * (p.I / 64) + ch / 2;
                        sc[l][c] = reinterpret_cast<const uint16_t*>(base + p.s_off[2])[g];
                        bi[l][c] = reinterpret_cast<const uint16_t*>(base + p.b_off[2])[g];
                    } else {
                        sc[l][c] = base[p.s_off[2] + static_cast<int64_t>(r) * (p.I / 32) + ch];
                        bi[l][c] = 0;
                    }
                }
            }
            uint64_t masks[4];
            pair_masks(p, e, lane, masks);
            for (int pr = next_pair(masks); pr >= 0; pr = next_pair(masks)) {
                const int t = pr / p.k;
                const float wt = p.w[pr];
                float hv[NC][32];
                float hs[NC];
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int ch = ch0 + c * WAVE;
                    const float4* hp =
                        reinterpret_cast<const float4*>(p.h + static_cast<int64_t>(pr) * p.I + ch * 32);
                    hs[c] = 0.0f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        float4 v = hp[i];
                        hv[c][4 * i + 0] = v.x;
                        hv[c][4 * i + 1] = v.y;
                        hv[c][4 * i + 2] = v.z;
                        hv[c][4 * i + 3] = v.w;
                        hs[c] += (v.x + v.y) + (v.z + v.w);
                    }
                }
#pragma unroll
                for (int l = 0; l < LOADS; ++l) {
                    float a = 0.0f;
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        const uint32_t d4[4] = {wgt[l][c].x, wgt[l][c].y, wgt[l][c].z, wgt[l][c].w};
                        float dq = 0.0f;
                        if (FMT == MOE355_W_INT4_G64) {
#pragma unroll
                            for (int d = 0; d < 4; ++d) {
                                const uint32_t lo = d4[d] & 0x0F0F0F0Fu;
                                const uint32_t hi = (d4[d] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
                                for (int b = 0; b < 4; ++b) {
                                    dq = fmaf(static_cast<float>((lo >> (8 * b)) & 0xFFu), hv[c][8 * d + 2 * b], dq);
                                    dq = fmaf(static_cast<float>((hi >> (8 * b)) & 0xFFu), hv[c][8 * d + 2 * b + 1], dq);
                                }
                            }
                            const float s = bf16_to_f32(static_cast<uint16_t>(sc[l][c]));
                            const float b = bf16_to_f32(static_cast<uint16_t>(bi[l][c]));
                            a += fmaf(s, dq, b * hs[c]);
                        } else {
#pragma unroll
                            for (int d = 0; d < 4; ++d) {
                                float2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d4[d], 1.0f, 0);
                                float2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d4[d], 1.0f, 1);
                                float2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d4[d], 1.0f, 2);
                                float2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d4[d], 1.0f, 3);
                                dq = fmaf(v0.x, hv[c][8 * d + 0], dq);
                                dq = fmaf(v0.y, hv[c][8 * d + 1], dq);
                                dq = fmaf(v1.x, hv[c][8 * d + 2], dq);
                                dq = fmaf(v1.y, hv[c][8 * d + 3], dq);
                                dq = fmaf(v2.x, hv[c][8 * d + 4], dq);
                                dq = fmaf(v2.y, hv[c][8 * d + 5], dq);
                                dq = fmaf(v3.x, hv[c][8 * d + 6], dq);
                                dq = fmaf(v3.y, hv[c][8 * d + 7], dq);
                            }
                            a += e8m0_to_f32(sc[l][c]) * dq;
                        }
                    }
                    a = segment_sum_f32(a, seg);
                    if (ch0 == 0) acc_lds[t * item_rows + rl0 + l * rpw] += wt * a;
                }
            }
        }
        __syncthreads();
        for (int i = threadIdx.x; i < p.T * item_rows; i += blockDim.x) {
            const int t = i / item_rows, rl = i - t * item_rows;
            p.out[static_cast<int64_t>(t) * p.H + item * item_rows + rl] = acc_lds[i];
        }
        __syncthreads();
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
    return L == 128 || L == 256 || L == 512 || L == 1024 || (L >= 2048 && L % 2048 == 0 && L <= 8192);
}

int device_cus() {
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        hipDeviceProp_t prop;
        if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
            cus = prop.multiProcessorCount;
        if (cus <= 0) cus = 256;
    }
    return cus;
}

template <int FMT>
moe355_status launch_decode(const DecodeParams& p, int max_uniq, hipStream_t stream) {
    int seg_h, nc_h, seg_i, nc_i;
    row_geometry(p.H, &seg_h, &nc_h);
    row_geometry(p.I, &seg_i, &nc_i);
    const int cus = device_cus();

    // gate/up: LOADS row loads per wavefront per item, so an item holds
    // 4 * LOADS * rpw rows of I
    {
        const int rpw = WAVE / seg_h;
        constexpr int LOADS = 4;
        const int item_rows = 4 * LOADS * rpw;
        MOE355_REQUIRE(p.I % item_rows == 0, MOE355_ENOTSUP, "decode: I=%d not a multiple of %d",
                       p.I, item_rows);
        const int items = max_uniq * (p.I / item_rows);
        const int grid = items < cus * 8 ? items : cus * 8;
        switch (nc_h) {
            case 1: gate_up_kernel<FMT, 1, LOADS, 2><<<grid, 256, 0, stream>>>(p, seg_h); break;
            case 2: gate_up_kernel<FMT, 2, LOADS, 2><<<grid, 256, 0, stream>>>(p, seg_h); break;
            case 4: gate_up_kernel<FMT, 4, LOADS, 1><<<grid, 256, 0, stream>>>(p, seg_h); break;
            default: return fail(MOE355_ENOTSUP, "decode: H=%d", p.H);
        }
        moe355_status st = check_launch("expert_ffn_decode gate_up");
        if (st) return st;
    }
    {
        const int rpw = WAVE / seg_i;
        constexpr int LOADS = 2;
        const int item_rows = 4 * LOADS * rpw;
        MOE355_REQUIRE(p.H % item_rows == 0, MOE355_ENOTSUP, "decode: H=%d not a multiple of %d",
                       p.H, item_rows);
        const size_t lds = static_cast<size_t>(p.T) * item_rows * sizeof(float);
        MOE355_REQUIRE(lds <= 64 * 1024, MOE355_ENOTSUP, "decode: T=%d too large for the combine",
                       p.T);
        const int items = p.H / item_rows;
        const int grid = items < cus * 8 ? items : cus * 8;
        switch (nc_i) {
            case 1: down_kernel<FMT, 1, LOADS><<<grid, 256, lds, stream>>>(p, seg_i); break;
            case 2: down_kernel<FMT, 2, LOADS><<<grid, 256, lds, stream>>>(p, seg_i); break;
            case 4: down_kernel<FMT, 4, LOADS><<<grid, 256, lds, stream>>>(p, seg_i); break;
            default: return fail(MOE355_ENOTSUP, "decode: I=%d", p.I);
        }
        return check_launch("expert_ffn_decode down");
    }
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
    MOE355_REQUIRE(T >= 0 && T * d->top_k <= 256, MOE355_ENOTSUP,
                   "expert_ffn_decode: T*k=%d outside [0, 256]", T * d->top_k);
    MOE355_REQUIRE(valid_row_len(d->hidden) && valid_row_len(d->inter), MOE355_ENOTSUP,
                   "expert_ffn_decode: H=%d I=%d unsupported", d->hidden, d->inter);
    if (T == 0) return ok();
    MOE355_REQUIRE(x_bf16 && topk_ids && topk_w && pool && exp && exp->uniq && exp->counts && out,
                   MOE355_EINVAL, "expert_ffn_decode: null pointer");
    const size_t need = moe355_workspace_bytes(d, T, MOE355_MODE_DECODE);
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
    p.h = static_cast<float*>(ws);
    p.out = out;
    if (cache) {
        MOE355_REQUIRE(cache->slot_table && cache->slot_data && cache->slot_bytes == L.bytes &&
                           cache->n_experts == d->n_experts && layer >= 0 &&
                           layer < cache->n_layers,
                       MOE355_EINVAL, "expert_ffn_decode: cache does not match the layer");
        p.table = cache->slot_table;
        p.slots = cache->slot_data;
    } else {
        MOE355_REQUIRE(layer >= 0, MOE355_EINVAL, "expert_ffn_decode: layer=%d", layer);
    }
    const int max_uniq = T * d->top_k < d->n_experts ? T * d->top_k : d->n_experts;
    if (d->wfmt == MOE355_W_INT4_G64) return launch_decode<MOE355_W_INT4_G64>(p, max_uniq, stream);
    return launch_decode<MOE355_W_MXFP4>(p, max_uniq, stream);
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
