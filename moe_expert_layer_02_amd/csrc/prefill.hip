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
//   * int4 (f16 MFMA): the weight operand is s * (q - 8), exact in f16 for any
//     bf16 scale because |q - 8| <= 8 keeps the product within 11 significant
//     bits; x is converted to f16 (exact for bf16 values in f16's range).  The
//     bias part sum_g (b + 8 s)[n, g] * sum_{c in g} x_c runs as a few extra
//     MFMAs over hi/lo f16 splits of both factors.
//   * MXFP4 (bf16 MFMA): e2m1 * 2^(e-127) is exact in bf16 (gfx950 converts
//     with the scale) and x is bf16 already.
//   * down projection: h = silu(g) * u enters as two 16-bit terms (hi + lo)
//     accumulated into the same registers.
//   * combine: out[t] += w * y with fp32 atomics in the down kernel's epilogue
//     (the gate/up kernel zeroes `out` first), so no [T*k, H] intermediate.
//
// Tiling: v_mfma_f32_32x32x16 (f16 for int4, bf16 for MXFP4), 4 wavefronts per
// block, tiles of 128 pair rows x 256 weight rows, K staged 64 at a time through
// double-buffered XOR-swizzled LDS with one barrier per stage; the next stage's
// global loads are issued before the current stage's MFMAs and dequantised into
// the other buffer after them.  Blocks are persistent (one per CU); the tiles of
// a call are split into 8 contiguous ranges, one per XCD (block id mod 8), so
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
    const uint16_t* xf;      // int4: [T][H] x as f16 in the int4 operand order
    const float* xsum;       // int4: [T][H / 64] group sums of x
    uint16_t* h_hi;          // [T*k][I] h = silu(g) * u, high half (f16 int4, bf16 MXFP4)
    uint16_t* h_lo;          // [T*k][I] remainder
    float* hsum;             // int4: [T*k][I / 64] group sums of h
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
// Shared pieces of the two GEMMs.  Block tile: 128 pair rows x 256 weight rows,
// K staged 64 at a time in double-buffered, XOR-swizzled LDS (one barrier per
// stage); wavefront (wm, wn) of the 2 x 2 grid computes 64 x 128 of it with 2 x 4
// MFMA 32x32 tiles.

constexpr int BN = 256;     // weight rows per tile

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

template <int FMT>
__device__ __forceinline__ f32x16 mma(uint4 a, uint4 b, f32x16 c) {
    if (FMT == MOE355_W_INT4_G64)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                      __builtin_bit_cast(half8, b), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pk_f16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}
__device__ __forceinline__ half2v as_h2(uint32_t v) { return __builtin_bit_cast(half2v, v); }

// int4: 8 codes of a dword as f16(s * (q - 8)) in the order (0,4,1,5,2,6,3,7),
// exact for any bf16 scale (|q - 8| <= 8 keeps the product within 11 bits).
__device__ __forceinline__ uint4 int4_dword_f16(uint32_t d, half2v s2) {
    const half2v off = {static_cast<_Float16>(-1032.0f), static_cast<_Float16>(-1032.0f)};
    uint32_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const half2v q = as_h2(((d >> (4 * i)) & 0x000F000Fu) | 0x64006400u);  // 1024 + q
        v[i] = __builtin_bit_cast(uint32_t, (q + off) * s2);
    }
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// 8 bf16 activations (natural order) as f16 in the int4 order above; adds their sum.
__device__ __forceinline__ uint4 x8_f16(uint4 v, float* sum) {
    const half2v one = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
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

__device__ __forceinline__ float f16x8_sum(uint4 v, float s) {
    const half2v one = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
    s = __builtin_amdgcn_fdot2(as_h2(v.x), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(v.y), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(v.z), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(v.w), one, s, false);
    return s;
}

// One staging thread's weight row for one stage: 64 codes, its scale(s).
struct WRow {
    uint4 q[2];
    uint32_t sc;   // int4: bf16 scale of the group; MXFP4: the two e8m0 bytes
};

template <int FMT>
__device__ __forceinline__ WRow load_wrow(const uint8_t* W, const PrefillParams& p, int m,
                                          int row, int kdim, int kk) {
    WRow r;
    const uint8_t* q = W + p.q_off[m] + static_cast<int64_t>(row) * (kdim / 2) + kk * 32;
    r.q[0] = reinterpret_cast<const uint4*>(q)[0];
    r.q[1] = reinterpret_cast<const uint4*>(q)[1];
    if (FMT == MOE355_W_INT4_G64)
        r.sc = reinterpret_cast<const uint16_t*>(W + p.s_off[m])[static_cast<int64_t>(row) * (kdim / 64) + kk];
    else
        r.sc = reinterpret_cast<const uint16_t*>(W + p.s_off[m] + static_cast<int64_t>(row) * (kdim / 32))[kk];
    return r;
}

// Dequantise one staged row into 8 LDS chunks (exact values: f16 for int4, bf16 for MXFP4).
template <int FMT>
__device__ __forceinline__ void store_wrow(uint4* Bs, int r, const WRow& w) {
    const uint32_t d[8] = {w.q[0].x, w.q[0].y, w.q[0].z, w.q[0].w,
                           w.q[1].x, w.q[1].y, w.q[1].z, w.q[1].w};
    if (FMT == MOE355_W_INT4_G64) {
        const _Float16 sh = static_cast<_Float16>(__uint_as_float(w.sc << 16));
        const half2v s2 = {sh, sh};
#pragma unroll
        for (int c = 0; c < 8; ++c) Bs[swz(r, c)] = int4_dword_f16(d[c], s2);
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const uint32_t e = (w.sc >> (8 * (c >> 2))) & 0xFFu;   // chunks 0-3: block 0
            const float sc = e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
            Bs[swz(r, c)] = make_uint4(
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[c], sc, 0)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[c], sc, 1)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[c], sc, 2)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[c], sc, 3)));
        }
    }
}

// The bias MFMA operands for 8 groups [g0, g0+8): b' = b + 8 s of weight row n
// as an f16 hi/lo pair (B side), and 8 group sums of one A row (A side).
__device__ __forceinline__ void bias_b(const uint8_t* W, const PrefillParams& p, int m, int n,
                                       int G, int g0, uint4* hi, uint4* lo) {
    // rows of b and s are G bf16 values (G even); 8 groups from g0 (a multiple of 8)
    const uint16_t* bp = reinterpret_cast<const uint16_t*>(W + p.b_off[m]) + static_cast<int64_t>(n) * G + g0;
    const uint16_t* sp = reinterpret_cast<const uint16_t*>(W + p.s_off[m]) + static_cast<int64_t>(n) * G + g0;
    uint32_t bw[4] = {0u, 0u, 0u, 0u}, sw[4] = {0u, 0u, 0u, 0u};
    if (g0 + 8 <= G) {
        const uint4 b4 = *reinterpret_cast<const uint4*>(bp), s4 = *reinterpret_cast<const uint4*>(sp);
        bw[0] = b4.x; bw[1] = b4.y; bw[2] = b4.z; bw[3] = b4.w;
        sw[0] = s4.x; sw[1] = s4.y; sw[2] = s4.z; sw[3] = s4.w;
    } else {
        // a short row (G = 2 or 4 groups, always even): only the dwords inside it
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (g0 + 2 * j < G) {
                bw[j] = reinterpret_cast<const uint32_t*>(bp)[j];
                sw[j] = reinterpret_cast<const uint32_t*>(sp)[j];
            }
        }
    }
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float v0 = __uint_as_float(bw[i] << 16) + 8.0f * __uint_as_float(sw[i] << 16);
        const float v1 = __uint_as_float(bw[i] & 0xFFFF0000u) + 8.0f * __uint_as_float(sw[i] & 0xFFFF0000u);
        const _Float16 a = static_cast<_Float16>(v0), b = static_cast<_Float16>(v1);
        h[i] = __builtin_bit_cast(uint32_t, half2v{a, b});
        l[i] = __builtin_bit_cast(uint32_t, half2v{static_cast<_Float16>(v0 - static_cast<float>(a)),
                                                  static_cast<_Float16>(v1 - static_cast<float>(b))});
    }
    *hi = make_uint4(h[0], h[1], h[2], h[3]);
    *lo = make_uint4(l[0], l[1], l[2], l[3]);
}
__device__ __forceinline__ void bias_a(const float* sums, int G, int g0, uint4* hi, uint4* lo) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = g0 + i < G ? sums[g0 + i] : 0.0f;
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const _Float16 a = static_cast<_Float16>(v[2 * i]), b = static_cast<_Float16>(v[2 * i + 1]);
        h[i] = __builtin_bit_cast(uint32_t, half2v{a, b});
        l[i] = __builtin_bit_cast(uint32_t, half2v{static_cast<_Float16>(v[2 * i] - static_cast<float>(a)),
                                                  static_cast<_Float16>(v[2 * i + 1] - static_cast<float>(b))});
    }
    *hi = make_uint4(h[0], h[1], h[2], h[3]);
    *lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// ---------------------------------------------------------------------------
// int4 pre-pass: x as f16 in the int4 operand order (exact for bf16 in f16's
// range) and its sums over each 64-wide group, once per call instead of once
// per tile.  A thread converts 8 values; 8 neighbouring threads form a group.
__global__ void __launch_bounds__(256) x16_kernel(const uint16_t* __restrict__ x, int64_t n8, int G,
                                                  uint16_t* __restrict__ xf, float* __restrict__ xsum) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // chunk of 8
    float s = 0.0f;
    if (i < n8) {
        const uint4 v = reinterpret_cast<const uint4*>(x)[i];
        reinterpret_cast<uint4*>(xf)[i] = x8_f16(v, &s);
    }
    s += __shfl_xor(s, 1, WAVE);
    s += __shfl_xor(s, 2, WAVE);
    s += __shfl_xor(s, 4, WAVE);
    if (i < n8 && (i & 7) == 0) xsum[i >> 3] = s;   // G groups per row, rows of H = 64 G
    (void)G;
}

// ---------------------------------------------------------------------------
// The GEMM pipeline shared by gate/up and down.  A (activation rows) travels
// global -> LDS by direct loads into a ring of PD stages, in the swizzled layout
// (lane i of a load lands at +16 i, so each lane fetches the chunk that belongs
// there); B (weight rows) travels global -> registers, PD stages ahead, straight
// in MFMA operand order, and is dequantised just before its MFMAs.  Wavefront w
// computes all 128 rows x 64 weight rows (two 32-wide column tiles).  Within a
// 64-wide stage, lane half hh holds inputs [32 hh, 32 hh + 32) and MFMA step s
// takes inputs 32 hh + 8 s + [0, 8) from both operands.

constexpr int PD = 3;        // stages in flight

typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ lds_ptr_t to_lds(const void* q) {
    return (lds_ptr_t)(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(q)));
}

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One stage of one lane's weight rows: 16 bytes of codes per column tile and its scale.
struct BRaw {
    uint4 q[2];
    uint32_t sc[2];   // int4: bf16 scale of the group; MXFP4: e8m0 of this lane's 32 inputs
};

// B operand of MFMA step s for one column tile.
template <int FMT>
__device__ __forceinline__ uint4 b_operand(const uint4& q, uint32_t sc, int s) {
    const uint32_t d = s == 0 ? q.x : s == 1 ? q.y : s == 2 ? q.z : q.w;
    if (FMT == MOE355_W_INT4_G64) {
        const _Float16 sh = static_cast<_Float16>(__uint_as_float(sc << 16));
        return int4_dword_f16(d, half2v{sh, sh});
    }
    const float scale = sc ? __uint_as_float(sc << 23) : __uint_as_float(0x00400000u);
    return make_uint4(
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 0)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 1)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 2)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 3)));
}

// A operand of MFMA step s for row tile mt from a staged 128 x 64 tile.
__device__ __forceinline__ uint4 a_operand(const uint4* A, int mt, int ln, int hh, int s) {
    const int r = mt * 32 + ln, c = 4 * hh + s;
    return A[r * 8 + (c ^ (r & 7))];
}

// Weight-row pointers of one lane for matrix m, row n, reduction length kdim.
template <int FMT>
struct BRow {
    const uint8_t* q;
    const uint8_t* s;
    __device__ void init(const uint8_t* W, const PrefillParams& p, int m, int n, int kdim, int hh) {
        q = W + p.q_off[m] + static_cast<int64_t>(n) * (kdim / 2) + hh * 16;
        s = FMT == MOE355_W_INT4_G64 ? W + p.s_off[m] + static_cast<int64_t>(n) * (kdim / 32)
                                     : W + p.s_off[m] + static_cast<int64_t>(n) * (kdim / 32) + hh;
    }
    __device__ void load(int kk, uint4* qv, uint32_t* sc) const {
        *qv = *reinterpret_cast<const uint4*>(q + kk * 32);
        *sc = FMT == MOE355_W_INT4_G64 ? reinterpret_cast<const uint16_t*>(s)[kk] : s[2 * kk];
    }
};

// ---------------------------------------------------------------------------
// gate/up: A = the tile's 128 gathered token rows (int4: the f16 copy of x),
// B = gate and up rows of features [f0 + 32 w, +32) for wavefront w.  Writes
// h = silu(g) * u as a hi/lo 16-bit pair, and for int4 the group sums of h.
template <int FMT>
__global__ void __launch_bounds__(256) gate_up_mfma(PrefillParams p) {
    extern __shared__ uint4 smem[];
    uint4* ring = smem;                                           // [PD][128 x 8 chunks]
    int32_t* rtok = reinterpret_cast<int32_t*>(smem + PD * 1024); // token of each tile row
    float* part = reinterpret_cast<float*>(rtok + BM);            // [4][64] h sums (int4)
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;
    const int ln = lane & 31, hh = lane >> 5;
    const int H = p.H, G = H / 64, KS = H / BK;

    {   // zero the layer output for the down kernel's atomics
        const int64_t n = static_cast<int64_t>(p.T) * H;
        for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + tid; i < n;
             i += static_cast<int64_t>(gridDim.x) * 256)
            p.out[i] = 0.0f;
    }

    const int FX = p.I / 128;
    const TileRange tr = tile_range(*p.n_tiles * FX);
    const uint16_t* xs = FMT == MOE355_W_INT4_G64 ? p.xf : p.x;
    for (int t = tr.begin; t < tr.end; t += tr.step) {
        const int y = t / FX, f0 = (t - y * FX) * 128;
        const int e = p.tile_e[y], m0 = p.tile_m0[y];
        const int pbase = p.offsets[e] + m0;
        const int rows = min(BM, p.offsets[e + 1] - pbase);
        const uint8_t* W = p.W + static_cast<int64_t>(e) * p.S;
        __syncthreads();   // the previous tile is done with the LDS
        // rows past the bucket re-read its first row (their outputs are dropped)
        if (tid < BM) rtok[tid] = p.perm[pbase + (tid < rows ? tid : 0)] / p.k;
        __syncthreads();
        int aoff[4];   // this lane's direct-load sources: 4 blocks of 8 rows of the tile
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 8 * (4 * wv + j) + lane / 8, c = (lane % 8) ^ (lane / 8);
            aoff[j] = rtok[r] * H + c * 8;
        }
        BRow<FMT> brow[2];
        brow[0].init(W, p, 0, f0 + 32 * wv + ln, H, hh);   // gate
        brow[1].init(W, p, 1, f0 + 32 * wv + ln, H, hh);   // up

        f32x16 R[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i) R[i][0] = R[i][1] = f32x16{};
        BRaw braw[PD];
        auto issue = [&](int kk, int slot, BRaw& b) {
            uint4* dst = ring + slot * 1024 + 4 * wv * 64;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                __builtin_amdgcn_global_load_lds(xs + aoff[j] + kk * BK, to_lds(dst + j * 64), 16, 0, 0);
            brow[0].load(kk, &b.q[0], &b.sc[0]);
            brow[1].load(kk, &b.q[1], &b.sc[1]);
        };
        auto compute = [&](int slot, const BRaw& b) {
            const uint4* A = ring + slot * 1024;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint4 b0 = b_operand<FMT>(b.q[0], b.sc[0], s);
                const uint4 b1 = b_operand<FMT>(b.q[1], b.sc[1], s);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const uint4 a = a_operand(A, mt, ln, hh, s);
                    R[mt][0] = mma<FMT>(a, b0, R[mt][0]);
                    R[mt][1] = mma<FMT>(a, b1, R[mt][1]);
                }
            }
        };
        issue(0, 0, braw[0]);
        if (KS > 1) issue(1, 1, braw[1]);
        for (int kb = 0; kb < KS; kb += PD) {
#pragma unroll
            for (int d = 0; d < PD; ++d) {
                const int kk = kb + d;
                if (kk < KS) {
                    // this stage's loads are done once only the next stage's 8 remain
                    if (kk + 1 < KS) wait_vm<8>();
                    else wait_vm<0>();
                    __syncthreads();
                    if (kk + 2 < KS) issue(kk + 2, (d + 2) % PD, braw[(d + 2) % PD]);
                    compute(d, braw[d]);
                }
            }
        }

        if (FMT == MOE355_W_INT4_G64) {
            // bias: R += sum_g xsum[m, g] * (b + 8 s)[n, g], both factors as f16 hi + lo
            for (int g0 = 0; g0 < G; g0 += 16) {
                const int gl = g0 + 8 * hh;
                uint4 bh[2], bl[2];
                bias_b(W, p, 0, f0 + 32 * wv + ln, G, gl, &bh[0], &bl[0]);
                bias_b(W, p, 1, f0 + 32 * wv + ln, G, gl, &bh[1], &bl[1]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    uint4 xh, xl;
                    bias_a(p.xsum + static_cast<int64_t>(rtok[mt * 32 + ln]) * G, G, gl, &xh, &xl);
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) {
                        R[mt][ct] = mma<FMT>(xh, bh[ct], R[mt][ct]);
                        R[mt][ct] = mma<FMT>(xl, bh[ct], R[mt][ct]);
                        R[mt][ct] = mma<FMT>(xh, bl[ct], R[mt][ct]);
                    }
                }
            }
        }

        // h = silu(g) * u as hi + lo 16-bit values, 64 rows at a time through the
        // ring (each wavefront its own 32 columns), stored as 16-byte row pieces
        __syncthreads();   // every wavefront is done reading the ring
        uint16_t* th = reinterpret_cast<uint16_t*>(ring) + wv * (2 * 64 * 32);   // [64][32] hi
        uint16_t* tl = th + 64 * 32;                                              // lo
        // int4: the down GEMM's operand order inside blocks of 8 columns
        const int col = FMT == MOE355_W_INT4_G64 ? (ln & ~7) + 2 * (ln & 3) + ((ln >> 2) & 1) : ln;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int mq = 0; mq < 2; ++mq) {
                const int mt = 2 * half + mq;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int rl = mq * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
                    const float g = R[mt][0][i], u = R[mt][1][i];
                    const float hv = g / (1.0f + __expf(-g)) * u;
                    uint16_t hi, lo;
                    if (FMT == MOE355_W_INT4_G64) {
                        const _Float16 a = static_cast<_Float16>(hv);
                        hi = __builtin_bit_cast(uint16_t, a);
                        lo = __builtin_bit_cast(uint16_t, static_cast<_Float16>(hv - static_cast<float>(a)));
                    } else {
                        const __bf16 a = static_cast<__bf16>(hv);
                        hi = __builtin_bit_cast(uint16_t, a);
                        lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(hv - static_cast<float>(a)));
                    }
                    th[rl * 32 + col] = hi;
                    tl[rl * 32 + col] = lo;
                }
            }
            __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wavefront's region only
            // 64 rows x 64 bytes per half: 4 pieces of 16 bytes per row
#pragma unroll
            for (int q = lane; q < 256; q += WAVE) {
                const int rl = q >> 2, c = q & 3, r = half * 64 + rl;
                if (r < rows) {
                    const int64_t at = static_cast<int64_t>(pbase + r) * p.I + f0 + 32 * wv + 8 * c;
                    *reinterpret_cast<uint4*>(p.h_hi + at) = reinterpret_cast<const uint4*>(th + rl * 32)[c];
                    *reinterpret_cast<uint4*>(p.h_lo + at) = reinterpret_cast<const uint4*>(tl + rl * 32)[c];
                }
            }
            if (FMT == MOE355_W_INT4_G64) {
                // this wavefront's share of each row's group sum (32 of a group's 64 columns)
                float sum = 0.0f;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    sum = f16x8_sum(reinterpret_cast<const uint4*>(th + lane * 32)[c], sum);
                    sum = f16x8_sum(reinterpret_cast<const uint4*>(tl + lane * 32)[c], sum);
                }
                part[wv * 64 + lane] = sum;
                __syncthreads();
                if ((wv & 1) == 0) {
                    const int r = half * 64 + lane;
                    if (r < rows)
                        p.hsum[static_cast<int64_t>(pbase + r) * (p.I / 64) + f0 / 64 + wv / 2] =
                            part[wv * 64 + lane] + part[(wv + 1) * 64 + lane];
                }
            }
            __syncthreads();   // the ring region is rewritten by the next half
        }
    }
}

// ---------------------------------------------------------------------------
// down + combine: A = the tile's 128 rows of h (hi and lo), B = down rows
// [n0 + 64 w, +64) for wavefront w; the weighted rows are added into the
// output with fp32 atomics.
template <int FMT>
__global__ void __launch_bounds__(256) down_mfma(PrefillParams p) {
    extern __shared__ uint4 smem[];
    uint4* ring = smem;                                           // [PD][hi 128 x 8, lo 128 x 8]
    int32_t* rtok = reinterpret_cast<int32_t*>(smem + PD * 2048);
    float* rw = reinterpret_cast<float*>(rtok + BM);
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;
    const int ln = lane & 31, hh = lane >> 5;
    const int I = p.I, Gd = I / 64, KS = I / BK;
    const int FX = p.H / BN;
    const TileRange tr = tile_range(*p.n_tiles * FX);
    for (int t = tr.begin; t < tr.end; t += tr.step) {
        const int y = t / FX, n0 = (t - y * FX) * BN;
        const int e = p.tile_e[y], m0 = p.tile_m0[y];
        const int pbase = p.offsets[e] + m0;
        const int rows = min(BM, p.offsets[e + 1] - pbase);
        const uint8_t* W = p.W + static_cast<int64_t>(e) * p.S;
        __syncthreads();   // the previous tile is done with the LDS
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
        int aoff[4];   // h rows are the bucket's pairs, contiguous from pbase
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 8 * (4 * wv + j) + lane / 8, c = (lane % 8) ^ (lane / 8);
            aoff[j] = (pbase + (r < rows ? r : 0)) * I + c * 8;
        }
        BRow<FMT> brow[2];
        brow[0].init(W, p, 2, n0 + 64 * wv + ln, I, hh);
        brow[1].init(W, p, 2, n0 + 64 * wv + 32 + ln, I, hh);

        f32x16 R[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i) R[i][0] = R[i][1] = f32x16{};
        BRaw braw[PD];
        auto issue = [&](int kk, int slot, BRaw& b) {
            uint4* dst = ring + slot * 2048 + 4 * wv * 64;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                __builtin_amdgcn_global_load_lds(p.h_hi + aoff[j] + kk * BK, to_lds(dst + j * 64), 16, 0, 0);
                __builtin_amdgcn_global_load_lds(p.h_lo + aoff[j] + kk * BK, to_lds(dst + 1024 + j * 64), 16, 0, 0);
            }
            brow[0].load(kk, &b.q[0], &b.sc[0]);
            brow[1].load(kk, &b.q[1], &b.sc[1]);
        };
        auto compute = [&](int slot, const BRaw& b) {
            const uint4* Ah = ring + slot * 2048;
            const uint4* Al = Ah + 1024;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint4 b0 = b_operand<FMT>(b.q[0], b.sc[0], s);
                const uint4 b1 = b_operand<FMT>(b.q[1], b.sc[1], s);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const uint4 ah = a_operand(Ah, mt, ln, hh, s);
                    const uint4 al = a_operand(Al, mt, ln, hh, s);
                    R[mt][0] = mma<FMT>(ah, b0, R[mt][0]);
                    R[mt][1] = mma<FMT>(ah, b1, R[mt][1]);
                    R[mt][0] = mma<FMT>(al, b0, R[mt][0]);
                    R[mt][1] = mma<FMT>(al, b1, R[mt][1]);
                }
            }
        };
        issue(0, 0, braw[0]);
        if (KS > 1) issue(1, 1, braw[1]);
        for (int kb = 0; kb < KS; kb += PD) {
#pragma unroll
            for (int d = 0; d < PD; ++d) {
                const int kk = kb + d;
                if (kk < KS) {
                    // this stage's loads are done once only the next stage's 12 remain
                    if (kk + 1 < KS) wait_vm<12>();
                    else wait_vm<0>();
                    __syncthreads();
                    if (kk + 2 < KS) issue(kk + 2, (d + 2) % PD, braw[(d + 2) % PD]);
                    compute(d, braw[d]);
                }
            }
        }

        if (FMT == MOE355_W_INT4_G64) {
            for (int g0 = 0; g0 < Gd; g0 += 16) {
                const int gl = g0 + 8 * hh;
                uint4 bh[2], bl[2];
                bias_b(W, p, 2, n0 + 64 * wv + ln, Gd, gl, &bh[0], &bl[0]);
                bias_b(W, p, 2, n0 + 64 * wv + 32 + ln, Gd, gl, &bh[1], &bl[1]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const int r = mt * 32 + ln;
                    uint4 xh, xl;
                    bias_a(p.hsum + static_cast<int64_t>(pbase + (r < rows ? r : 0)) * Gd, Gd, gl, &xh, &xl);
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) {
                        R[mt][ct] = mma<FMT>(xh, bh[ct], R[mt][ct]);
                        R[mt][ct] = mma<FMT>(xl, bh[ct], R[mt][ct]);
                        R[mt][ct] = mma<FMT>(xh, bl[ct], R[mt][ct]);
                    }
                }
            }
        }

        // combine: out[t, n] += w * y
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = mt * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
                if (r < rows) {
                    const float wt = rw[r];
                    float* orow = p.out + static_cast<int64_t>(rtok[r]) * p.H + n0 + 64 * wv + ln;
                    unsafeAtomicAdd(orow, wt * R[mt][0][i]);
                    unsafeAtomicAdd(orow + 32, wt * R[mt][1][i]);
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
        blocks = ((cus + NXCD - 1) / NXCD) * NXCD;   // one resident block per CU
    }
    return blocks;
}

}  // namespace

// h (hi, lo), the tile plan, the tile count, and for int4 the f16 copy of x,
// its group sums and the group sums of h.
size_t prefill_ws_bytes(const moe355_layer_desc* d, int T) {
    const size_t tk = static_cast<size_t>(T) * d->top_k;
    const size_t xb = d->wfmt == MOE355_W_INT4_G64
                          ? align256(static_cast<size_t>(T) * d->hidden * 2) +
                                align256(static_cast<size_t>(T) * (d->hidden / 64) * 4) +
                                align256(tk * (d->inter / 64) * 4)
                          : 0;
    return align256(tk * d->inter * sizeof(float)) +
           align256(2 * static_cast<size_t>(max_tiles(T, d->top_k, d->n_experts)) * sizeof(int32_t)) +
           256 + xb;
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
    MOE355_REQUIRE(d->hidden % 256 == 0 && d->inter % 128 == 0 && d->n_experts <= 1024,
                   MOE355_ENOTSUP, "expert_ffn_prefill: H=%d (multiple of 256), I=%d (of 128), E=%d",
                   d->hidden, d->inter, d->n_experts);
    MOE355_REQUIRE(d->hidden <= 8192 && d->inter <= 2048, MOE355_ENOTSUP,
                   "expert_ffn_prefill: H=%d (at most 8192) or I=%d (at most 2048) too large for LDS",
                   d->hidden, d->inter);
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
    p.h_hi = reinterpret_cast<uint16_t*>(wsb);
    p.h_lo = p.h_hi + tk * d->inter;
    const size_t off_tiles = align256(tk * d->inter * sizeof(float));
    const int mt = max_tiles(T, d->top_k, d->n_experts);
    int32_t* tiles = reinterpret_cast<int32_t*>(wsb + off_tiles);
    p.tile_e = tiles;
    p.tile_m0 = tiles + mt;
    p.n_tiles = reinterpret_cast<int32_t*>(wsb + off_tiles + align256(2 * static_cast<size_t>(mt) * 4));
    p.out = out;
    const size_t off_x = off_tiles + align256(2 * static_cast<size_t>(mt) * 4) + 256;
    uint16_t* xf = reinterpret_cast<uint16_t*>(wsb + off_x);
    float* xsum = reinterpret_cast<float*>(wsb + off_x + align256(static_cast<size_t>(T) * d->hidden * 2));
    p.xf = xf;
    p.xsum = xsum;
    p.hsum = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(xsum) +
                                      align256(static_cast<size_t>(T) * (d->hidden / 64) * 4));

    plan_kernel<<<1, 1024, 0, stream>>>(offsets, d->n_experts, tiles, tiles + mt,
                                        const_cast<int32_t*>(p.n_tiles));
    st = check_launch("expert_ffn_prefill plan");
    if (st) return st;
    const int blocks = prefill_blocks();
    const bool int4 = d->wfmt == MOE355_W_INT4_G64;
    if (int4) {
        const int64_t n8 = static_cast<int64_t>(T) * d->hidden / 8;
        x16_kernel<<<static_cast<unsigned>((n8 + 255) / 256), 256, 0, stream>>>(
            p.x, n8, d->hidden / 64, xf, xsum);
        st = check_launch("expert_ffn_prefill x16");
        if (st) return st;
    }
    const size_t lds_gu = PD * 16384 + BM * 4 + 4 * 64 * 4;
    const size_t lds_dn = PD * 32768 + 2 * BM * 4;
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
