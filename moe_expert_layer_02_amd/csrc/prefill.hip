// Prefill expert FFN: a grouped GEMM over each expert's token bucket on the
// CDNA4 matrix cores, with the whole layer resident.
//
// [Edge0, section 3.1 "Executor paths"]: for prefill the whole layer's experts
// are loaded at once and each expert runs over the tokens routed to it;
// [Edge0, section 3.1 "Math contract"]: y = down(silu(gate(x)) * up(x));
// [FT-zh, Core method]: the outputs of a token's experts merge into one sum.
//
// Precision scheme (the layer output must stay within 2e-2 absolute of an exact
// evaluation while int4-g64 outputs reach several hundred):
//   * x is bf16, so it is an exact MFMA operand.
//   * int4: the B operand is the nibble q itself (exact in bf16).  Each 64-wide
//     K step is one quantisation group, so its MFMA partial P_g is scaled by
//     s[n, g] in fp32 on the VALU; the bias part sum_g b[n, g] * sum_{c in g} x_c
//     runs as a small extra MFMA over the group sums split into two bf16 terms.
//   * MXFP4: e2m1 * 2^(e-127) is exact in bf16 (gfx950 converts with the scale),
//     so one MFMA per step and no epilogue.
//   * down projection: h = silu(g) * u is fp32; it enters the MFMA as two bf16
//     terms (h_hi + h_lo) accumulated into the same registers.
//   * combine: out[t] += w * y with fp32 atomics in the down kernel's epilogue
//     (the gate/up kernel zeroes `out` first), so no [T*k, H] intermediate.
//
// Tiling: v_mfma_f32_32x32x16_bf16, 4 wavefronts per block, 128 pair rows per
// tile, K staged 64 at a time through XOR-swizzled LDS, next step's global loads
// issued before the current step's MFMAs.  Blocks are persistent; the tiles of a
// call are split into 8 contiguous ranges, one per XCD (block id mod 8), so
// tiles that share activation rows or an expert's weights share an L2.
#include "internal.h"

namespace moe355 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128;     // pair rows per tile
constexpr int BK = 64;      // K per stage (one int4 group, two MXFP4 blocks)
constexpr int NXCD = 8;

struct PrefillParams {
    const uint16_t* x;
    const int32_t* perm;
    const int32_t* offsets;
    const float* topk_w;
    const uint8_t* W;
    int64_t S;
    int64_t q_off[3], s_off[3], b_off[3];
    int T, k, H, I, E;
    const int32_t* tile_e;
    const int32_t* tile_m0;
    const int32_t* n_tiles;
    float* h;
    float* out;
};

__device__ __forceinline__ f32x16 mfma(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2 v;
    v.x = static_cast<__bf16>(lo);
    v.y = static_cast<__bf16>(hi);
    return __builtin_bit_cast(uint32_t, v);
}

// 8 consecutive fp32 values as hi and lo bf16 parts (v = hi + lo to ~16 bits).
__device__ __forceinline__ void split8(const float* v, uint4& hi, uint4& lo) {
    float h[8], l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        h[i] = static_cast<float>(static_cast<__bf16>(v[i]));
        l[i] = v[i] - h[i];
    }
    hi = make_uint4(pack_bf16(h[0], h[1]), pack_bf16(h[2], h[3]), pack_bf16(h[4], h[5]),
                    pack_bf16(h[6], h[7]));
    lo = make_uint4(pack_bf16(l[0], l[1]), pack_bf16(l[2], l[3]), pack_bf16(l[4], l[5]),
                    pack_bf16(l[6], l[7]));
}

// 32 int4 nibbles (16 bytes, element 2c = low nibble of byte c) -> 32 exact bf16.
__device__ __forceinline__ void nibbles_to_bf16(uint4 q, uint4 out[4]) {
    const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = d[i] & 0x0F0F0F0Fu, hi = (d[i] >> 4) & 0x0F0F0F0Fu;
        float f[8];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            f[2 * b] = static_cast<float>((lo >> (8 * b)) & 0xFFu);
            f[2 * b + 1] = static_cast<float>((hi >> (8 * b)) & 0xFFu);
        }
        // small integers are exact in bf16: the top half of the fp32 pattern
        out[i] = make_uint4(
            (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xFFFF0000u),
            (__float_as_uint(f[2]) >> 16) | (__float_as_uint(f[3]) & 0xFFFF0000u),
            (__float_as_uint(f[4]) >> 16) | (__float_as_uint(f[5]) & 0xFFFF0000u),
            (__float_as_uint(f[6]) >> 16) | (__float_as_uint(f[7]) & 0xFFFF0000u));
    }
}

// 32 e2m1 codes (one MX block) times 2^(e-127) -> 32 exact bf16.
__device__ __forceinline__ void fp4_to_bf16(uint4 q, uint32_t e, uint4 out[4]) {
    const float sc = e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
    const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[i] = make_uint4(
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], sc, 0)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], sc, 1)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], sc, 2)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], sc, 3)));
    }
}

__device__ __forceinline__ float bf16_sum8(uint4 v) {
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s += __uint_as_float(d[i] << 16) + __uint_as_float(d[i] & 0xFFFF0000u);
    return s;
}

// LDS tile of 128 rows x 64 bf16, 16-byte chunk c of row r at (c ^ (r & 7)).
__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ (r & 7)); }

// Persistent tile loop: the work of a call split into NXCD contiguous ranges.
struct TileRange {
    int begin, end, step;
};
__device__ __forceinline__ TileRange tile_range(int total) {
    const int xcd = blockIdx.x % NXCD;
    const int per = gridDim.x / NXCD;
    TileRange r;
    r.begin = static_cast<int>(static_cast<int64_t>(total) * xcd / NXCD) + blockIdx.x / NXCD;
    r.end = static_cast<int>(static_cast<int64_t>(total) * (xcd + 1) / NXCD);
    r.step = per;
    return r;
}

// ---------------------------------------------------------------------------
// Tile plan: tile j covers rows [tile_m0[j], +BM) of expert tile_e[j]'s bucket.
__global__ void __launch_bounds__(1024) plan_kernel(const int32_t* __restrict__ offsets, int E,
                                                    int32_t* __restrict__ tile_e,
                                                    int32_t* __restrict__ tile_m0,
                                                    int32_t* __restrict__ n_tiles) {
    __shared__ int32_t wave_tot[16];
    const int e = threadIdx.x, lane = e & (WAVE - 1), w = e / WAVE;
    const int me = e < E ? offsets[e + 1] - offsets[e] : 0;
    const int nt = (me + BM - 1) / BM;
    int inc = nt;
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
        int o = __shfl_up(inc, d, WAVE);
        if (lane >= d) inc += o;
    }
    if (lane == WAVE - 1) wave_tot[w] = inc;
    __syncthreads();
    int base = 0, all = 0;
    for (int i = 0; i < 16; ++i) {
        if (i < w) base += wave_tot[i];
        all += wave_tot[i];
    }
    base += inc - nt;
    for (int i = 0; i < nt; ++i) {
        tile_e[base + i] = e;
        tile_m0[base + i] = i * BM;
    }
    if (e == 0) *n_tiles = all;
}

// ---------------------------------------------------------------------------
// gate/up: tile = 128 pair rows x 64 features (64 gate + 64 up weight rows).
// Wavefront (wm, wf) owns rows [64 wm, +64) and features [32 wf, +32).
template <int FMT>
__global__ void __launch_bounds__(256) gate_up_mfma(PrefillParams p) {
    extern __shared__ uint4 smem[];
    uint4* As = smem;                                  // 128 x 64 bf16
    uint4* Bs = smem + 1024;                           // 128 x 64 bf16
    float* Xg = reinterpret_cast<float*>(smem + 2048); // [128][G] group sums (int4)
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;
    const int wm = wv >> 1, wf = wv & 1;
    const int H = p.H, G = H / 64, KS = H / BK;

    {   // zero the layer output for the down kernel's atomics
        const int64_t n = static_cast<int64_t>(p.T) * H;
        for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + tid; i < n;
             i += static_cast<int64_t>(gridDim.x) * 256)
            p.out[i] = 0.0f;
    }

    const int FX = p.I / 64;
    const TileRange tr = tile_range(*p.n_tiles * FX);
    const int ar = tid >> 1, ah = tid & 1;             // staging row / half
    for (int t = tr.begin; t < tr.end; t += tr.step) {
        const int y = t / FX, f0 = (t - y * FX) * 64;
        const int e = p.tile_e[y], m0 = p.tile_m0[y];
        const int pbase = p.offsets[e] + m0;
        const int rows = min(BM, p.offsets[e + 1] - pbase);
        const uint8_t* W = p.W + static_cast<int64_t>(e) * p.S;
        const int tok = ar < rows ? p.perm[pbase + ar] / p.k : -1;
        const uint16_t* xrow = tok >= 0 ? p.x + static_cast<int64_t>(tok) * H + ah * 32 : nullptr;
        const int bm = ar < 64 ? 0 : 1;                // B staging row: gate or up
        const int brow = f0 + (ar & 63);
        const uint8_t* bq = W + p.q_off[bm] + static_cast<int64_t>(brow) * (H / 2) + ah * 16;
        const uint8_t* be = W + p.s_off[bm] + static_cast<int64_t>(brow) * (H / 32) + ah;

        f32x16 R[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) R[i][j] = f32x16{};

        uint4 a_next[4], b_next;
        uint32_t e_next = 0;
        auto load_stage = [&](int kk) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                a_next[c] = xrow ? reinterpret_cast<const uint4*>(xrow + kk * BK)[c]
                                 : make_uint4(0, 0, 0, 0);
            b_next = *reinterpret_cast<const uint4*>(bq + kk * 32);
            if (FMT == MOE355_W_MXFP4) e_next = be[kk * 2];
        };
        load_stage(0);
        const int n_lane = f0 + wf * 32 + (lane & 31);  // feature of this lane's accumulators
        for (int kk = 0; kk < KS; ++kk) {
            __syncthreads();
            {   // stage kk into LDS
                uint4 bc[4];
                if (FMT == MOE355_W_INT4_G64) nibbles_to_bf16(b_next, bc);
                else fp4_to_bf16(b_next, e_next, bc);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    As[swz(ar, ah * 4 + c)] = a_next[c];
                    Bs[swz(ar, ah * 4 + c)] = bc[c];
                }
                if (FMT == MOE355_W_INT4_G64) {
                    float xs = bf16_sum8(a_next[0]) + bf16_sum8(a_next[1]) + bf16_sum8(a_next[2]) +
                               bf16_sum8(a_next[3]);
                    xs += __shfl_xor(xs, 1, WAVE);
                    if (ah == 0) Xg[ar * G + kk] = xs;
                }
            }
            __syncthreads();
            if (kk + 1 < KS) load_stage(kk + 1);
            float sg = 0.0f, su = 0.0f;
            if (FMT == MOE355_W_INT4_G64) {
                sg = bf16_to_f32(reinterpret_cast<const uint16_t*>(W + p.s_off[0])[n_lane * G + kk]);
                su = bf16_to_f32(reinterpret_cast<const uint16_t*>(W + p.s_off[1])[n_lane * G + kk]);
            }
            f32x16 P[2][2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) P[i][j] = FMT == MOE355_W_INT4_G64 ? f32x16{} : R[i][j];
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) {
                const int c = 2 * k4 + (lane >> 5);
                uint4 af[2], bf[2];
#pragma unroll
                for (int ms = 0; ms < 2; ++ms) {
                    const int r = wm * 64 + ms * 32 + (lane & 31);
                    af[ms] = As[swz(r, c)];
                }
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    const int r = g * 64 + wf * 32 + (lane & 31);
                    bf[g] = Bs[swz(r, c)];
                }
#pragma unroll
                for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                    for (int g = 0; g < 2; ++g) P[ms][g] = mfma(af[ms], bf[g], P[ms][g]);
            }
#pragma unroll
            for (int ms = 0; ms < 2; ++ms) {
                if (FMT == MOE355_W_INT4_G64) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        R[ms][0][i] = fmaf(sg, P[ms][0][i], R[ms][0][i]);
                        R[ms][1][i] = fmaf(su, P[ms][1][i], R[ms][1][i]);
                    }
                } else {
                    R[ms][0] = P[ms][0];
                    R[ms][1] = P[ms][1];
                }
            }
        }

        if (FMT == MOE355_W_INT4_G64) {
            __syncthreads();  // Xg complete
            // bias: R += sum_g Xg[m, g] * b[n, g], Xg as bf16 hi + lo
            for (int g0 = 0; g0 < G; g0 += 16) {
                const int gl = g0 + 8 * (lane >> 5);
                uint4 bb[2];
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    const uint16_t* bp = reinterpret_cast<const uint16_t*>(W + p.b_off[g]) +
                                         static_cast<int64_t>(n_lane) * G + gl;
                    uint32_t v[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t lo = gl + 2 * i < G ? bp[2 * i] : 0u;
                        const uint32_t hi = gl + 2 * i + 1 < G ? bp[2 * i + 1] : 0u;
                        v[i] = lo | (hi << 16);
                    }
                    bb[g] = make_uint4(v[0], v[1], v[2], v[3]);
                }
#pragma unroll
                for (int ms = 0; ms < 2; ++ms) {
                    const int r = wm * 64 + ms * 32 + (lane & 31);
                    float xv[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) xv[i] = gl + i < G ? Xg[r * G + gl + i] : 0.0f;
                    uint4 xh, xl;
                    split8(xv, xh, xl);
#pragma unroll
                    for (int g = 0; g < 2; ++g) {
                        R[ms][g] = mfma(xh, bb[g], R[ms][g]);
                        R[ms][g] = mfma(xl, bb[g], R[ms][g]);
                    }
                }
            }
        }

        // h = silu(g) * u for the tile's valid rows
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = wm * 64 + ms * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                if (r < rows) {
                    const float g = R[ms][0][i], u = R[ms][1][i];
                    p.h[static_cast<int64_t>(pbase + r) * p.I + n_lane] = g / (1.0f + __expf(-g)) * u;
                }
            }
    }
}

// ---------------------------------------------------------------------------
// down + combine: tile = 128 pair rows x 128 outputs; wavefront (wm, wn) owns
// rows [64 wm, +64) and outputs [64 wn, +64).
template <int FMT>
__global__ void __launch_bounds__(256) down_mfma(PrefillParams p) {
    extern __shared__ uint4 smem[];
    uint4* Ah = smem;                                   // h hi, 128 x 64 bf16
    uint4* Al = smem + 1024;                            // h lo
    uint4* Bs = smem + 2048;                            // W_down rows, 128 x 64 bf16
    int32_t* rtok = reinterpret_cast<int32_t*>(smem + 3072);  // token of each tile row
    float* rw = reinterpret_cast<float*>(rtok + BM);          // its routing weight
    float* Hg = rw + BM;                                      // [128][Gd] group sums (int4)
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;
    const int wm = wv >> 1, wn = wv & 1;
    const int I = p.I, Gd = I / 64, KS = I / BK;
    const int FX = p.H / 128;
    const TileRange tr = tile_range(*p.n_tiles * FX);
    const int ar = tid >> 1, ah = tid & 1;
    for (int t = tr.begin; t < tr.end; t += tr.step) {
        const int y = t / FX, n0 = (t - y * FX) * 128;
        const int e = p.tile_e[y], m0 = p.tile_m0[y];
        const int pbase = p.offsets[e] + m0;
        const int rows = min(BM, p.offsets[e + 1] - pbase);
        const uint8_t* W = p.W + static_cast<int64_t>(e) * p.S;
        __syncthreads();   // previous tile's readers of rtok / rw are done
        if (tid < BM) {
            if (tid < rows) {
                const int pr = p.perm[pbase + tid];
                rtok[tid] = pr / p.k;
                rw[tid] = p.topk_w[pr];
            } else {
                rtok[tid] = -1;
                rw[tid] = 0.0f;
            }
        }
        const float* hrow = ar < rows ? p.h + static_cast<int64_t>(pbase + ar) * I + ah * 32 : nullptr;
        const int brow = n0 + ar;
        const uint8_t* bq = W + p.q_off[2] + static_cast<int64_t>(brow) * (I / 2) + ah * 16;
        const uint8_t* be = W + p.s_off[2] + static_cast<int64_t>(brow) * (I / 32) + ah;

        f32x16 R[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) R[i][j] = f32x16{};
        float4 a_next[8];
        uint4 b_next;
        uint32_t e_next = 0;
        auto load_stage = [&](int kk) {
#pragma unroll
            for (int c = 0; c < 8; ++c)
                a_next[c] = hrow ? reinterpret_cast<const float4*>(hrow + kk * BK)[c]
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
            b_next = *reinterpret_cast<const uint4*>(bq + kk * 32);
            if (FMT == MOE355_W_MXFP4) e_next = be[kk * 2];
        };
        load_stage(0);
        int n_lane[2];
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) n_lane[ns] = n0 + wn * 64 + ns * 32 + (lane & 31);
        for (int kk = 0; kk < KS; ++kk) {
            __syncthreads();
            {
                uint4 bc[4];
                if (FMT == MOE355_W_INT4_G64) nibbles_to_bf16(b_next, bc);
                else fp4_to_bf16(b_next, e_next, bc);
                float hs = 0.0f;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float v[8] = {a_next[2 * c].x, a_next[2 * c].y, a_next[2 * c].z,
                                        a_next[2 * c].w, a_next[2 * c + 1].x, a_next[2 * c + 1].y,
                                        a_next[2 * c + 1].z, a_next[2 * c + 1].w};
                    uint4 hi, lo;
                    split8(v, hi, lo);
                    Ah[swz(ar, ah * 4 + c)] = hi;
                    Al[swz(ar, ah * 4 + c)] = lo;
                    Bs[swz(ar, ah * 4 + c)] = bc[c];
                    if (FMT == MOE355_W_INT4_G64)
#pragma unroll
                        for (int i = 0; i < 8; ++i) hs += v[i];
                }
                if (FMT == MOE355_W_INT4_G64) {
                    hs += __shfl_xor(hs, 1, WAVE);
                    if (ah == 0) Hg[ar * Gd + kk] = hs;
                }
            }
            __syncthreads();
            if (kk + 1 < KS) load_stage(kk + 1);
            float sc[2] = {0.0f, 0.0f};
            if (FMT == MOE355_W_INT4_G64)
#pragma unroll
                for (int ns = 0; ns < 2; ++ns)
                    sc[ns] = bf16_to_f32(
                        reinterpret_cast<const uint16_t*>(W + p.s_off[2])[n_lane[ns] * Gd + kk]);
            f32x16 P[2][2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) P[i][j] = FMT == MOE355_W_INT4_G64 ? f32x16{} : R[i][j];
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) {
                const int c = 2 * k4 + (lane >> 5);
                uint4 afh[2], afl[2], bf[2];
#pragma unroll
                for (int ms = 0; ms < 2; ++ms) {
                    const int r = wm * 64 + ms * 32 + (lane & 31);
                    afh[ms] = Ah[swz(r, c)];
                    afl[ms] = Al[swz(r, c)];
                }
#pragma unroll
                for (int ns = 0; ns < 2; ++ns) {
                    const int r = wn * 64 + ns * 32 + (lane & 31);
                    bf[ns] = Bs[swz(r, c)];
                }
#pragma unroll
                for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                    for (int ns = 0; ns < 2; ++ns) {
                        P[ms][ns] = mfma(afh[ms], bf[ns], P[ms][ns]);
                        P[ms][ns] = mfma(afl[ms], bf[ns], P[ms][ns]);
                    }
            }
#pragma unroll
            for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                for (int ns = 0; ns < 2; ++ns) {
                    if (FMT == MOE355_W_INT4_G64) {
#pragma unroll
                        for (int i = 0; i < 16; ++i) R[ms][ns][i] = fmaf(sc[ns], P[ms][ns][i], R[ms][ns][i]);
                    } else {
                        R[ms][ns] = P[ms][ns];
                    }
                }
        }

        if (FMT == MOE355_W_INT4_G64) {
            __syncthreads();  // Hg complete
            for (int g0 = 0; g0 < Gd; g0 += 16) {
                const int gl = g0 + 8 * (lane >> 5);
                uint4 bb[2];
#pragma unroll
                for (int ns = 0; ns < 2; ++ns) {
                    const uint16_t* bp = reinterpret_cast<const uint16_t*>(W + p.b_off[2]) +
                                         static_cast<int64_t>(n_lane[ns]) * Gd + gl;
                    uint32_t v[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t lo = gl + 2 * i < Gd ? bp[2 * i] : 0u;
                        const uint32_t hi = gl + 2 * i + 1 < Gd ? bp[2 * i + 1] : 0u;
                        v[i] = lo | (hi << 16);
                    }
                    bb[ns] = make_uint4(v[0], v[1], v[2], v[3]);
                }
#pragma unroll
                for (int ms = 0; ms < 2; ++ms) {
                    const int r = wm * 64 + ms * 32 + (lane & 31);
                    float hv[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) hv[i] = gl + i < Gd ? Hg[r * Gd + gl + i] : 0.0f;
                    uint4 hh, hl;
                    split8(hv, hh, hl);
#pragma unroll
                    for (int ns = 0; ns < 2; ++ns) {
                        R[ms][ns] = mfma(hh, bb[ns], R[ms][ns]);
                        R[ms][ns] = mfma(hl, bb[ns], R[ms][ns]);
                    }
                }
            }
        }

        // combine: out[t, n] += w * y
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = wm * 64 + ms * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                if (r < rows) {
                    const int tk = rtok[r];
                    const float wt = rw[r];
                    float* orow = p.out + static_cast<int64_t>(tk) * p.H;
#pragma unroll
                    for (int ns = 0; ns < 2; ++ns) unsafeAtomicAdd(orow + n_lane[ns], wt * R[ms][ns][i]);
                }
            }
    }
}

int max_tiles(int T, int k, int E) { return (T * k + BM - 1) / BM + E; }

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

int prefill_blocks() {
    static int blocks = 0;
    if (!blocks) {
        int dev = 0, cus = 0;
        hipDeviceProp_t prop;
        if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
            cus = prop.multiProcessorCount;
        if (cus <= 0) cus = 256;
        blocks = ((cus * 2 + NXCD - 1) / NXCD) * NXCD;   // two resident blocks per CU
    }
    return blocks;
}

}  // namespace

size_t prefill_ws_bytes(const moe355_layer_desc* d, int T) {
    const size_t tk = static_cast<size_t>(T) * d->top_k;
    return align256(tk * d->inter * sizeof(float)) +
           align256(2 * static_cast<size_t>(max_tiles(T, d->top_k, d->n_experts)) * sizeof(int32_t)) +
           256;
}

}  // namespace moe355

using namespace moe355;

extern "C" moe355_status moe355_expert_ffn_prefill(const moe355_layer_desc* d, const void* x_bf16,
                                                   int32_t T, const int32_t* topk_ids,
                                                   const float* topk_w, const uint8_t* layer_w,
                                                   const int32_t* perm, const int32_t* offsets,
                                                   float* out, void* ws, size_t ws_bytes,
                                                   hipStream_t stream) {
    (void)topk_ids;
    moe355_status st = check_desc(d);
    if (st) return st;
    MOE355_REQUIRE(T >= 0 && static_cast<int64_t>(T) * d->top_k < (1ll << 28), MOE355_EINVAL,
                   "expert_ffn_prefill: T=%d", T);
    if (T == 0) return ok();
    MOE355_REQUIRE(x_bf16 && topk_w && layer_w && perm && offsets && out, MOE355_EINVAL,
                   "expert_ffn_prefill: null pointer");
    MOE355_REQUIRE(d->hidden % 128 == 0 && d->inter % 64 == 0 && d->n_experts <= 1024,
                   MOE355_ENOTSUP, "expert_ffn_prefill: H=%d (multiple of 128), I=%d (of 64), E=%d",
                   d->hidden, d->inter, d->n_experts);
    MOE355_REQUIRE(d->hidden / 64 <= 256 && d->inter / 64 <= 128, MOE355_ENOTSUP,
                   "expert_ffn_prefill: H or I too large for the LDS group sums");
    const size_t need = prefill_ws_bytes(d, T);
    MOE355_REQUIRE(ws && ws_bytes >= need, MOE355_ECAPACITY,
                   "expert_ffn_prefill: workspace %zu < %zu bytes", ws_bytes, need);
    ExpertLayout L;
    expert_layout(d, &L);
    const size_t tk = static_cast<size_t>(T) * d->top_k;
    uint8_t* wsb = static_cast<uint8_t*>(ws);
    PrefillParams p{};
    p.x = static_cast<const uint16_t*>(x_bf16);
    p.perm = perm;
    p.offsets = offsets;
    p.topk_w = topk_w;
    p.W = layer_w;
    p.S = L.bytes;
    for (int m = 0; m < 3; ++m) {
        p.q_off[m] = L.q_off[m];
        p.s_off[m] = L.s_off[m];
        p.b_off[m] = L.b_off[m];
    }
    p.T = T;
    p.k = d->top_k;
    p.H = d->hidden;
    p.I = d->inter;
    p.E = d->n_experts;
    p.h = reinterpret_cast<float*>(wsb);
    const size_t off_tiles = align256(tk * d->inter * sizeof(float));
    const int mt = max_tiles(T, d->top_k, d->n_experts);
    int32_t* tiles = reinterpret_cast<int32_t*>(wsb + off_tiles);
    p.tile_e = tiles;
    p.tile_m0 = tiles + mt;
    p.n_tiles = reinterpret_cast<int32_t*>(wsb + off_tiles + align256(2 * static_cast<size_t>(mt) * 4));
    p.out = out;

    plan_kernel<<<1, 1024, 0, stream>>>(offsets, d->n_experts, tiles, tiles + mt,
                                        const_cast<int32_t*>(p.n_tiles));
    st = check_launch("expert_ffn_prefill plan");
    if (st) return st;
    const int blocks = prefill_blocks();
    const bool int4 = d->wfmt == MOE355_W_INT4_G64;
    const size_t lds_gu = 2 * 16384 + (int4 ? static_cast<size_t>(BM) * (d->hidden / 64) * 4 : 0);
    const size_t lds_dn = 3 * 16384 + (int4 ? static_cast<size_t>(BM) * (d->inter / 64) * 4 : 0) +
                          2 * BM * 4;
    MOE355_REQUIRE(lds_gu <= 160 * 1024 && lds_dn <= 160 * 1024, MOE355_ENOTSUP,
                   "expert_ffn_prefill: LDS need %zu / %zu bytes", lds_gu, lds_dn);
    auto gu = int4 ? gate_up_mfma<MOE355_W_INT4_G64> : gate_up_mfma<MOE355_W_MXFP4>;
    auto dn = int4 ? down_mfma<MOE355_W_INT4_G64> : down_mfma<MOE355_W_MXFP4>;
    // raise the dynamic LDS limit once per kernel when a shape needs more than 64 KB
    static size_t granted[2][2] = {{64 * 1024, 64 * 1024}, {64 * 1024, 64 * 1024}};
    const int fi = int4 ? 0 : 1;
    if (lds_gu > granted[fi][0]) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(gu),
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                static_cast<int>(lds_gu)) != hipSuccess)
            return fail(MOE355_EHIP, "expert_ffn_prefill: LDS %zu bytes refused", lds_gu);
        granted[fi][0] = lds_gu;
    }
    if (lds_dn > granted[fi][1]) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(dn),
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                static_cast<int>(lds_dn)) != hipSuccess)
            return fail(MOE355_EHIP, "expert_ffn_prefill: LDS %zu bytes refused", lds_dn);
        granted[fi][1] = lds_dn;
    }
    gu<<<blocks, 256, lds_gu, stream>>>(p);
    st = check_launch("expert_ffn_prefill gate_up");
    if (st) return st;
    dn<<<blocks, 256, lds_dn, stream>>>(p);
    return check_launch("expert_ffn_prefill down");
}
