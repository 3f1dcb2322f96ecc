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
//   * combine: the down kernel stores each pair's y row (fp32, plain stores)
//     at row t k + j of a [T*k, H] workspace array; a last pass sums a token's
//     k rows with its weights, j ascending.  An fp32 atomic add per output
//     element would avoid the intermediate but runs at one element per L2
//     channel per clock, several times slower than the store and re-read.
//
// Tiling: v_mfma_f32_32x32x16 (f16 for int4, bf16 for MXFP4), 4 wavefronts per
// block, tiles of 128 pair rows x 256 weight rows, K staged 64 at a time through
// double-buffered XOR-swizzled LDS with one barrier per stage; the next stage's
// global loads are issued before the current stage's MFMAs and dequantised into
// the other buffer after them.  Blocks are persistent (one per CU); the tiles of
// a call are split into 8 contiguous ranges, one per XCD (block id mod 8), so
// tiles that share activation rows or an expert's weights share an L2.
#include <type_traits>

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
    float* y;                // [T*k][H] down outputs by pair id t k + j
    uint32_t* err;           // the call's error word (cleared by the plan kernel)
};

// A load of memory that no kernel of the launch writes (the tile plan, the
// bucket offsets) through the constant address space: at a wavefront-uniform
// address the compiler makes it a scalar load, whose wait (lgkmcnt) does not
// also wait for the vector-memory stores and direct loads in flight.
template <typename T>
__device__ __forceinline__ T ld_const(const T* q) {
    typedef const __attribute__((address_space(4))) T* ConstPtr;
    return *(ConstPtr)(q);
}

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
                                                    int32_t* __restrict__ n_tiles,
                                                    uint32_t* __restrict__ err) {
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
    if (e == 0) {
        *n_tiles = all;
        *err = 0u;
    }
}

// ---------------------------------------------------------------------------
// Shared pieces of the two GEMMs.

// An accumulator element read out of its AGPR at this point of the program.
// Left to itself the compiler copies all 256 accumulators of a tile to VGPRs
// right after the K loop, which spills other values (and a spill reload waits
// for every memory operation in flight, the next tile's loads included).  The
// caller guarantees that the MFMA that wrote the element finished (the
// epilogue starts with enough wait states, see mfma_drain).
__device__ __forceinline__ float acc_read(float a) {
    float v;
    asm("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}
// Wait states after the last MFMA before acc_read may read its result (more
// than a 16-pass MFMA needs).
__device__ __forceinline__ void mfma_drain() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// The values of lanes l and l ^ 32 by gfx950's v_permlane32_swap (a VALU op,
// no LDS round trip): lanes 0-31 get (v[l], v[l + 32]), lanes 32-63
// (v[l - 32], v[l]) (checked with a one-wavefront probe).
__device__ __forceinline__ uint32_t half_partner(uint32_t v, int hh) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return hh ? r[0] : r[1];
}
__device__ __forceinline__ float max_with_partner(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_partner(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// silu(g) = g / (1 + e^-g) with the hardware reciprocal (1 ulp); e^-g = inf
// gives -0 for very negative g.
__device__ __forceinline__ float silu(float g) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}


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
    // the two masks live in registers, so that (x & mask) | magic is one
    // v_and_or_b32 (gfx9 encodes at most one literal per VALU instruction)
    uint32_t mask = 0x000F000Fu, magic = 0x64006400u;
    asm("" : "+v"(mask), "+v"(magic));
    uint32_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const half2v q = as_h2(((d >> (4 * i)) & mask) | magic);  // 1024 + q
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

// The bias MFMA operands for 8 groups [g0, g0+8): b' = b + 8 s of weight row n
// as an f16 hi/lo pair (B side), and 8 group sums of one A row (A side).  In the
// device layout group g of row n sits in the scale (bias) word of block
// (n / 16, g / 2), half g % 2.
// Loads and conversions are separate calls, so that a tile issues all the
// loads of 16 groups before it waits for any (one round trip, not one per call).
struct BiasRaw {
    uint32_t bw[4], sw[4];   // B side: bias and scale words of 8 groups
    float x[8];              // A side: 8 group sums
};
__device__ __forceinline__ void bias_b_load(const uint8_t* W, const PrefillParams& p, int m, int n,
                                            int G, int g0, BiasRaw& r) {
    const int64_t row = static_cast<int64_t>(n / 16) * (G / 2) * 64 + (n & 15) * 4;
    const uint8_t* bp = W + p.b_off[m] + row;
    const uint8_t* sp = W + p.s_off[m] + row;
#pragma unroll
    for (int j = 0; j < 4; ++j) {   // groups past G read group 0 (zeroed by bias_b_cvt)
        const int64_t o = static_cast<int64_t>(g0 + 2 * j < G ? g0 / 2 + j : 0) * 64;
        r.bw[j] = *reinterpret_cast<const uint32_t*>(bp + o);
        r.sw[j] = *reinterpret_cast<const uint32_t*>(sp + o);
    }
}
// a short row (G = 2, 4 or 6 groups, always even) ends inside the 8
__device__ __forceinline__ void bias_b_cvt(const BiasRaw& r, int G, int g0, uint4* hi, uint4* lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool in = g0 + 2 * i < G;
        const uint32_t bw = in ? r.bw[i] : 0u, sw = in ? r.sw[i] : 0u;
        const float v0 = __uint_as_float(bw << 16) + 8.0f * __uint_as_float(sw << 16);
        const float v1 = __uint_as_float(bw & 0xFFFF0000u) + 8.0f * __uint_as_float(sw & 0xFFFF0000u);
        const _Float16 a = static_cast<_Float16>(v0), b = static_cast<_Float16>(v1);
        h[i] = __builtin_bit_cast(uint32_t, half2v{a, b});
        l[i] = __builtin_bit_cast(uint32_t, half2v{static_cast<_Float16>(v0 - static_cast<float>(a)),
                                                  static_cast<_Float16>(v1 - static_cast<float>(b))});
    }
    *hi = make_uint4(h[0], h[1], h[2], h[3]);
    *lo = make_uint4(l[0], l[1], l[2], l[3]);
}
// 8 group sums [g0, g0 + 8) of a row of G (even) sums, 8-byte loads; sums past
// G read sum 0 and are zeroed by bias_a_cvt.
__device__ __forceinline__ void bias_a_load(const float* sums, int G, int g0, BiasRaw& r) {
    const float2* s2 = reinterpret_cast<const float2*>(sums);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float2 v = s2[g0 + 2 * i < G ? g0 / 2 + i : 0];
        r.x[2 * i] = v.x;
        r.x[2 * i + 1] = v.y;
    }
}
__device__ __forceinline__ void bias_a_cvt(const BiasRaw& r, int G, int g0, uint4* hi, uint4* lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool in = g0 + 2 * i < G;
        const float x0 = in ? r.x[2 * i] : 0.0f, x1 = in ? r.x[2 * i + 1] : 0.0f;
        const _Float16 a = static_cast<_Float16>(x0), b = static_cast<_Float16>(x1);
        h[i] = __builtin_bit_cast(uint32_t, half2v{a, b});
        l[i] = __builtin_bit_cast(uint32_t, half2v{static_cast<_Float16>(x0 - static_cast<float>(a)),
                                                  static_cast<_Float16>(x1 - static_cast<float>(b))});
    }
    *hi = make_uint4(h[0], h[1], h[2], h[3]);
    *lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// ---------------------------------------------------------------------------
// int4 pre-pass: x as f16 in the int4 operand order (exact for bf16 in f16's
// range) and its sums over each 64-wide group, once per call instead of once
// per tile.  A thread converts 8 values; 8 neighbouring threads form a group.
__global__ void __launch_bounds__(256) x16_kernel(const uint16_t* __restrict__ x, int64_t n8, int G,
                                                  uint16_t* __restrict__ xf, float* __restrict__ xsum,
                                                  uint32_t* __restrict__ err) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // chunk of 8
    float s = 0.0f;
    if (i < n8) {
        const uint4 v = reinterpret_cast<const uint4*>(x)[i];
        reinterpret_cast<uint4*>(xf)[i] = x8_f16(v, &s);
        // a value beyond f16's range would not convert exactly: flag the call
        if (bf16_mag_beyond_f16(bf16_mag_max(v, u16x2_t{0, 0})))
            __hip_atomic_fetch_or(err, ERR_F16_RANGE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    s += __shfl_xor(s, 1, WAVE);
    s += __shfl_xor(s, 2, WAVE);
    s += __shfl_xor(s, 4, WAVE);
    if (i < n8 && (i & 7) == 0) xsum[i >> 3] = s;   // G groups per row, rows of H = 64 G
    (void)G;
}

// ---------------------------------------------------------------------------
// The GEMM pipeline shared by gate/up and down.  Both operands travel global ->
// LDS by direct loads (global_load_lds: lane i of a load lands 16 i bytes, or 4 i
// for a dword load, past the LDS address in M0) into a ring of PD stage slots,
// PD - 1 stages ahead of the MFMAs; one barrier per stage.
//   A (activation rows): 128 rows x 64 inputs; 16-byte chunk c of row r sits at
//     chunk (c ^ swz8(r)) of the row, so each lane fetches the chunk that belongs
//     where it lands and the MFMA reads are free of bank conflicts.
//   B (weight rows): per wavefront 2 column tiles x 64 lanes x 16 bytes of codes
//     in MFMA operand order, then one dword per lane and tile holding its scale.
// Within a stage, lane half hh holds inputs [32 hh, 32 hh + 32) and MFMA step s
// takes inputs 32 hh + 8 s + [0, 8) from both operands.
//
// The loads are issued from inline assembly.  The compiler's wait-count pass
// cannot tell the ring slots apart, so for its own form of these loads it waits
// for every one in flight before the first LDS read of a stage, which turns the
// ring into a fully serialised load -> compute sequence.  Hidden from it, the
// only waits on them are the explicit per-stage ones below (vector-memory
// operations of one wavefront complete in issue order, so "at most n in flight"
// means all but the last n loads have landed).

// A wavefront-uniform pointer held in scalar registers.
__device__ __forceinline__ const void* uniform_ptr(const void* q) {
    const uint64_t v = reinterpret_cast<uint64_t>(q);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Direct loads of base + voff (32-bit byte offset, per lane) into LDS at lds;
// base and lds are wavefront-uniform.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :: "v"(voff), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}

// Wait until at most N of this wavefront's loads are in flight and its LDS reads
// are done, then meet the other wavefronts.
template <int N>
__device__ __forceinline__ void stage_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
}
// The same with N = OPS * min(R, rem) for a runtime rem >= 0.
template <int OPS, int R>
__device__ __forceinline__ void stage_wait(int rem) {
    if constexpr (R == 0) {
        stage_barrier<0>();
    } else {
        if (rem >= R) stage_barrier<R * OPS>();
        else stage_wait<OPS, R - 1>(rem);
    }
}

__device__ __forceinline__ uint32_t lds_addr(const void* q) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(q));
}

// B operand of MFMA step s from one lane's 16 code bytes; sc is the lane's scale
// dword (int4: two bf16 group scales, kk odd takes the high one; MXFP4: four e8m0
// bytes, byte 2 (kk & 1) + hh is this lane's).
template <int FMT>
__device__ __forceinline__ uint4 b_operand(const uint4& q, uint32_t sc, int kk, int hh, int s) {
    const uint32_t d = s == 0 ? q.x : s == 1 ? q.y : s == 2 ? q.z : q.w;
    if (FMT == MOE355_W_INT4_G64) {
        const uint32_t b = (kk & 1) ? (sc & 0xFFFF0000u) : (sc << 16);
        const _Float16 sh = static_cast<_Float16>(__uint_as_float(b));
        return int4_dword_f16(d, half2v{sh, sh});
    }
    const uint32_t e = (sc >> (8 * (2 * (kk & 1) + hh))) & 0xFFu;
    const float scale = e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
    return make_uint4(
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 0)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 1)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 2)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 3)));
}

// LDS swizzles of staged activation rows.  A 16-byte read by 64 lanes is served
// 16 lanes (256 bytes, the LDS's 64 four-byte banks) at a time; the 16 lanes of
// a group read 16 consecutive rows at one chunk index, so a row's chunks are
// permuted to put those rows on distinct banks:
//   128-byte rows (8 chunks): chunk c at slot c ^ ((r >> 1) & 7) -- rows of one
//     parity share a 128-byte bank half and differ in (r >> 1) & 7;
//   64-byte rows (4 chunks): chunk c at slot c ^ ((r >> 2) & 3) -- four
//     consecutive rows fill 256 bytes and the next four move to other slots.
// (XOR with r & 7 or r & 3 puts rows r and r + 8, or r + 4, on the same banks:
// measured 1.2e8 and 1.7e8 bank-conflict cycles per call on the DS-like layer.)
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz4(int r) { return (r >> 2) & 3; }

// A operand of MFMA step s for row tile mt from a staged 128 x 64 tile.
__device__ __forceinline__ uint4 a_operand(const uint4* A, int mt, int ln, int hh, int s) {
    const int r = mt * 32 + ln, c = 4 * hh + s;
    return A[r * 8 + (c ^ swz8(r))];
}

// Byte offsets (from the expert's blob) of weight sources in the device
// layout, where each region is cut into blocks of 16 rows x 128 inputs (a code
// block of 1 KB holds chunk j of row r at (16 j + r) * 16; a scale block holds
// row r's word at 4 r).  A 64-input stage kk is half a block: chunks
// 2 (kk & 1) + {0, 1}, so lane half hh of row n reads chunk 2 (kk & 1) + hh of
// block (n / 16, kk / 2), and the word that covers the stage is the block's.
__device__ __forceinline__ uint32_t code_src(int64_t q_off, int n, int kdim, int hh) {
    return static_cast<uint32_t>(q_off + static_cast<int64_t>(n / 16) * (kdim / 128) * 1024 +
                                 (16 * hh + (n & 15)) * 16);
}
__device__ __forceinline__ uint32_t code_step(int kk) { return (kk >> 1) * 1024 + (kk & 1) * 512; }
__device__ __forceinline__ uint32_t scale_src(int64_t s_off, int n, int kdim) {
    return static_cast<uint32_t>(s_off + static_cast<int64_t>(n / 16) * (kdim / 128) * 64 + (n & 15) * 4);
}
__device__ __forceinline__ uint32_t scale_step(int kk) { return (kk >> 1) * 64; }

// Stage slot layouts (bytes).  gate/up: A = 128 rows x 64 inputs; B codes
// [wavefront][4 column tiles][64 lanes] x 16 bytes; scales [wavefront][2][64]
// dwords, load j holding the scale dwords of the wavefront's weight rows
// 64 j + [0, 64), so column tile c finds its row ln at 32 (c & 1) + ln of load c / 2.
constexpr int GU_A = 0, GU_B = 16384, GU_S = 32768, GU_SLOT = 34816, GU_PD = 4;
// down: A = hi and lo parts of 128 rows x 64 inputs of h; B as above.
constexpr int DN_AH = 0, DN_AL = 16384, DN_B = 32768, DN_S = 49152, DN_SLOT = 51200, DN_PD = 3;
constexpr int GU_FEAT = 256;   // features per gate/up tile: 64 per wavefront
constexpr int DN_COLS = 512;   // output columns per down tile: 128 per wavefront

// The scale dword of column tile c for this lane, from a slot's scale region.
__device__ __forceinline__ uint32_t tile_scale(const uint32_t* S, int wv, int c, int ln) {
    return S[(2 * wv + (c >> 1)) * 64 + 32 * (c & 1) + ln];
}

// ---------------------------------------------------------------------------
// gate/up: A = the tile's 128 gathered token rows (int4: the f16 copy of x); B =
// for wavefront w the gate rows (column tiles 0, 1) and up rows (tiles 2, 3) of
// features fw + [0, 64), fw = f0 + 64 w.  The MFMAs take the weights as their
// first operand, so an accumulator holds 32 features x 32 tokens and a lane holds
// runs of 4 consecutive features of one token: h = silu(g) * u leaves as 8-byte
// stores straight from registers (hi and lo 16-bit parts), and for int4 the
// group sums of h need one exchange between the lane halves.
template <int FMT>
__global__ void __launch_bounds__(256) gate_up_mfma(PrefillParams p) {
    constexpr int PD = GU_PD, OPS = 10;   // loads per stage per wavefront
    extern __shared__ uint4 smem[];
    uint8_t* ring = reinterpret_cast<uint8_t*>(smem);                  // [PD][GU_SLOT]
    int32_t* rtok = reinterpret_cast<int32_t*>(ring + PD * GU_SLOT);   // token of each tile row
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int H = p.H, I = p.I, G = H / 64, KS = H / BK;
    const uint32_t ring_lds = lds_addr(ring);

    const int FX = (I + GU_FEAT - 1) / GU_FEAT;
    const TileRange tr = tile_range(ld_const(p.n_tiles) * FX);
    const void* xs = uniform_ptr(FMT == MOE355_W_INT4_G64 ? p.xf : p.x);
    for (int t = tr.begin; t < tr.end; t += tr.step) {
        const int y = t / FX;
        const int e = ld_const(p.tile_e + y), m0 = ld_const(p.tile_m0 + y);
        const int pbase = ld_const(p.offsets + e) + m0;
        const int rows = min(BM, ld_const(p.offsets + e + 1) - pbase);
        const void* W = uniform_ptr(p.W + static_cast<int64_t>(e) * p.S);
        const int fw = (t - y * FX) * GU_FEAT + 64 * wv;
        // The lane index is made opaque once per tile so that the compiler
        // recomputes lane-derived addresses here instead of hoisting dozens of
        // them out of the tile loop (they would spill, and every reload of a
        // spill waits for all memory operations in flight).
        int lane = tid & (WAVE - 1);
        asm volatile("" : "+v"(lane));
        const int ln = lane & 31, hh = lane >> 5;
        const bool live = fw < I;            // the last tile of a small I may leave wavefronts idle
        const int fr = live ? fw : 0;        // (they compute on row 0 and store nothing)
        __syncthreads();   // the previous tile is done with the LDS
        // rows past the bucket re-read its first row (their outputs are dropped)
        if (tid < BM) rtok[tid] = p.perm[pbase + (tid < rows ? tid : 0)] / p.k;
        __syncthreads();
        uint32_t aoff[4];   // this lane's A sources: 4 blocks of 8 rows of the tile
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 8 * (4 * wv + j) + lane / 8, c = (lane % 8) ^ swz8(r);
            aoff[j] = static_cast<uint32_t>(rtok[r]) * static_cast<uint32_t>(2 * H) + c * 16;
        }
        uint32_t bq[4], bsc[2];
#pragma unroll
        for (int c = 0; c < 4; ++c) bq[c] = code_src(p.q_off[c >> 1], fr + 32 * (c & 1) + ln, H, hh);
#pragma unroll
        for (int j = 0; j < 2; ++j) bsc[j] = scale_src(p.s_off[j], fr + lane, H);

        f32x16 R[4][4];   // [column tile][row tile]
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) R[c][i] = f32x16{};
        // One stage's operands of a lane: A fragments [MFMA step][row tile], the
        // codes and scale dwords of the 4 column tiles.
        struct Ops {
            uint4 a[4][4];
            uint4 q[4];
            uint32_t sc[4];
        };
        // load i (of OPS) of stage kk into the slot at LDS address sl
        auto load_op = [&](int kk, uint32_t sl, int i) {
            if (i < 4) {
                dma16(xs, aoff[i] + kk * 128, sl + GU_A + (4 * wv + i) * 1024);
            } else if (i < 8) {
                dma16(W, bq[i - 4] + code_step(kk), sl + GU_B + (4 * wv + i - 4) * 1024);
            } else {
                dma4(W, bsc[i - 8] + scale_step(kk), sl + GU_S + (2 * wv + i - 8) * 256);
            }
        };
        // read piece i of a stage: 0..3 the codes and scale of column tile i,
        // then A fragment (s, mt) as piece 4 + 4 s + mt
        auto read_op = [&](const uint8_t* sp, int i, Ops& o) {
            if (i < 4) {
                o.q[i] = (reinterpret_cast<const uint4*>(sp + GU_B) + 4 * wv * 64 + lane)[i * 64];
                o.sc[i] = tile_scale(reinterpret_cast<const uint32_t*>(sp + GU_S), wv, i, ln);
            } else {
                const int s4 = (i - 4) >> 2, mt = (i - 4) & 3;
                o.a[s4][mt] = a_operand(reinterpret_cast<const uint4*>(sp + GU_A), mt, ln, hh, s4);
            }
        };
        // Iteration kk, as in gate_up_mx: the MFMAs of stage kk from cur (the
        // weight operand of each (step, column tile) dequantised in registers
        // one group ahead), between them the reads of stage kk + 1 into nxt and
        // the loads of stage kk + PD (the last stage again past the end).
        auto iter = [&](auto NMTc, int kk, int slot, const Ops& cur, Ops& nxt) {
            constexpr int NMT = decltype(NMTc)::value;
            constexpr int NP = 4 + 4 * NMT;   // pieces the next stage needs
            stage_barrier<OPS * (PD - 2)>();  // stage kk + 1 has landed everywhere
            const int nslot = slot == PD - 1 ? 0 : slot + 1;
            const uint8_t* spn = ring + nslot * GU_SLOT;
            const uint32_t sl = ring_lds + slot * GU_SLOT;
            const int kl = min(kk + PD, KS - 1);
            uint4 b[2];
            b[0] = b_operand<FMT>(cur.q[0], cur.sc[0], kk, hh, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int g = 0; g < 16; ++g) {   // group g: MFMA step g / 4, column tile g % 4
#pragma unroll
                for (int mt = 0; mt < NMT; ++mt) {
                    R[g & 3][mt] = mma<FMT>(b[g & 1], cur.a[g >> 2][mt], R[g & 3][mt]);
                    if (mt == 0 && g + 1 < 16)
                        b[(g + 1) & 1] = b_operand<FMT>(cur.q[(g + 1) & 3], cur.sc[(g + 1) & 3], kk, hh, (g + 1) >> 2);
                    const int j = g * NMT + mt;
#pragma unroll
                    for (int u = 2 * j; u < 2 * j + 2; ++u)
                        if (u < NP) read_op(spn, u < 4 ? u : 4 + 4 * ((u - 4) / NMT) + (u - 4) % NMT, nxt);
                    if (j >= 4 && j - 4 < OPS) load_op(kl, sl, j - 4);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        auto kloop = [&](auto NMTc) {
            constexpr int NMT = decltype(NMTc)::value;
            Ops o0, o1;
#pragma unroll
            for (int s4 = 0; s4 < PD; ++s4)
#pragma unroll
                for (int i = 0; i < OPS; ++i) load_op(s4 < KS ? s4 : KS - 1, ring_lds + s4 * GU_SLOT, i);
            stage_barrier<OPS * (PD - 1)>();   // stage 0 has landed everywhere
#pragma unroll
            for (int u = 0; u < 4 + 4 * NMT; ++u) read_op(ring, u < 4 ? u : 4 + 4 * ((u - 4) / NMT) + (u - 4) % NMT, o0);
            int slot = 0;
#pragma nounroll
            for (int kk = 0; kk < KS; kk += 2) {   // KS is even
                iter(NMTc, kk, slot, o0, o1);
                slot = slot == PD - 1 ? 0 : slot + 1;
                iter(NMTc, kk + 1, slot, o1, o0);
                slot = slot == PD - 1 ? 0 : slot + 1;
            }
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");   // the repeated loads have landed
        };
        switch (__builtin_amdgcn_readfirstlane((rows + 31) / 32)) {
            case 1: kloop(std::integral_constant<int, 1>{}); break;
            case 2: kloop(std::integral_constant<int, 2>{}); break;
            case 3: kloop(std::integral_constant<int, 3>{}); break;
            default: kloop(std::integral_constant<int, 4>{}); break;
        }

        if (FMT == MOE355_W_INT4_G64) {
            // bias: R += sum_g (b + 8 s)[n, g] * xsum[m, g], both factors as f16 hi + lo
            for (int g0 = 0; g0 < G; g0 += 16) {
                const int gl = g0 + 8 * hh, BG = G;
                BiasRaw rb[4], ra[4];   // every load of the 16 groups first, then one wait
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    bias_b_load(static_cast<const uint8_t*>(W), p, c >> 1, fr + 32 * (c & 1) + ln, G, gl, rb[c]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    bias_a_load(p.xsum + static_cast<int64_t>(rtok[mt * 32 + ln]) * G, G, gl, ra[mt]);
                uint4 bh[4], bl[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) bias_b_cvt(rb[c], BG, gl, &bh[c], &bl[c]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    uint4 xh, xl;
                    bias_a_cvt(ra[mt], BG, gl, &xh, &xl);
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        R[c][mt] = mma<FMT>(bh[c], xh, R[c][mt]);
                        R[c][mt] = mma<FMT>(bh[c], xl, R[c][mt]);
                        R[c][mt] = mma<FMT>(bl[c], xh, R[c][mt]);
                    }
                }
            }
        }

        mfma_drain();
        // h = silu(g) * u.  Lane (ln, hh) holds, for token row 32 mt + ln, features
        // fw + 32 ft + 8 q + 4 hh + [0, 4) in R[ft][mt][4 q + 0..3] (g) and R[2 + ft] (u).
        // int4 stores each block of 8 features in the down GEMM's operand order
        // (0, 4, 1, 5, 2, 6, 3, 7): lane half 0 writes positions 0-3 = features
        // 0, 4, 1, 5 and half 1 positions 4-7 = features 2, 6, 3, 7, after trading
        // features 2, 3 (half 0) for 4, 5 (half 1).
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int r = mt * 32 + ln;
            const bool keep = live && r < rows;
            const int64_t row = static_cast<int64_t>(pbase + r) * I;
            float gsum = 0.0f;
#pragma unroll
            for (int ft = 0; ft < 2; ++ft) {
                uint32_t HW[4][2], LW[4][2];   // per 8-feature block q: this lane's 4 values, hi and lo
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint32_t* hw = HW[q];
                    uint32_t* lw = LW[q];
                    uint16_t hi[4], lo[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float g = acc_read(R[ft][mt][4 * q + j]), u = acc_read(R[2 + ft][mt][4 * q + j]);
                        const float hv = silu(g) * u;
                        if (FMT == MOE355_W_INT4_G64) {
                            const _Float16 x1 = static_cast<_Float16>(hv);
                            const _Float16 x2 = static_cast<_Float16>(hv - static_cast<float>(x1));
                            hi[j] = __builtin_bit_cast(uint16_t, x1);
                            lo[j] = __builtin_bit_cast(uint16_t, x2);
                            gsum += static_cast<float>(x1) + static_cast<float>(x2);
                        } else {
                            const __bf16 x1 = static_cast<__bf16>(hv);
                            hi[j] = __builtin_bit_cast(uint16_t, x1);
                            lo[j] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(hv - static_cast<float>(x1)));
                        }
                    }
                    if (FMT == MOE355_W_INT4_G64) {
                        const uint32_t gh = hh ? (hi[0] | (static_cast<uint32_t>(hi[1]) << 16))
                                               : (hi[2] | (static_cast<uint32_t>(hi[3]) << 16));
                        const uint32_t gl = hh ? (lo[0] | (static_cast<uint32_t>(lo[1]) << 16))
                                               : (lo[2] | (static_cast<uint32_t>(lo[3]) << 16));
                        const uint32_t rh = half_partner(gh, hh), rl = half_partner(gl, hh);
                        if (hh == 0) {
                            hw[0] = hi[0] | (rh << 16);
                            hw[1] = hi[1] | (rh & 0xFFFF0000u);
                            lw[0] = lo[0] | (rl << 16);
                            lw[1] = lo[1] | (rl & 0xFFFF0000u);
                        } else {
                            hw[0] = (rh & 0xFFFFu) | (static_cast<uint32_t>(hi[2]) << 16);
                            hw[1] = (rh >> 16) | (static_cast<uint32_t>(hi[3]) << 16);
                            lw[0] = (rl & 0xFFFFu) | (static_cast<uint32_t>(lo[2]) << 16);
                            lw[1] = (rl >> 16) | (static_cast<uint32_t>(lo[3]) << 16);
                        }
                    } else {
                        hw[0] = hi[0] | (static_cast<uint32_t>(hi[1]) << 16);
                        hw[1] = hi[2] | (static_cast<uint32_t>(hi[3]) << 16);
                        lw[0] = lo[0] | (static_cast<uint32_t>(lo[1]) << 16);
                        lw[1] = lo[2] | (static_cast<uint32_t>(lo[3]) << 16);
                    }
                }
                // lane half 0 holds positions 0-3 of each block, half 1 positions
                // 4-7: half 0 trades its blocks 1, 3 for half 1's blocks 0, 2, and
                // each lane stores two whole blocks (16 bytes each) of hi and of lo
#pragma unroll
                for (int qq = 0; qq < 2; ++qq) {
                    const uint32_t rh0 = half_partner(hh ? HW[2 * qq][0] : HW[2 * qq + 1][0], hh);
                    const uint32_t rh1 = half_partner(hh ? HW[2 * qq][1] : HW[2 * qq + 1][1], hh);
                    const uint32_t rl0 = half_partner(hh ? LW[2 * qq][0] : LW[2 * qq + 1][0], hh);
                    const uint32_t rl1 = half_partner(hh ? LW[2 * qq][1] : LW[2 * qq + 1][1], hh);
                    if (keep) {
                        const int64_t at = row + fw + 32 * ft + 8 * (2 * qq + hh);
                        const uint4 vh = hh ? make_uint4(rh0, rh1, HW[2 * qq + 1][0], HW[2 * qq + 1][1])
                                            : make_uint4(HW[2 * qq][0], HW[2 * qq][1], rh0, rh1);
                        const uint4 vl = hh ? make_uint4(rl0, rl1, LW[2 * qq + 1][0], LW[2 * qq + 1][1])
                                            : make_uint4(LW[2 * qq][0], LW[2 * qq][1], rl0, rl1);
                        *reinterpret_cast<uint4*>(p.h_hi + at) = vh;
                        *reinterpret_cast<uint4*>(p.h_lo + at) = vl;
                    }
                }
            }
            if (FMT == MOE355_W_INT4_G64) {
                // the row's sum over the wavefront's 64 features: one int4 group of h
                // (not finite when an h value left f16's range: flag the call)
                gsum = sum_with_partner(gsum);
                if (keep && !(__builtin_fabsf(gsum) <= 3.0e38f))
                    __hip_atomic_fetch_or(p.err, ERR_F16_RANGE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (keep && hh == 0) p.hsum[static_cast<int64_t>(pbase + r) * (I / 64) + fw / 64] = gsum;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Down epilogue: accumulator R[mt][c] of a wavefront holds rows 32 mt + 8 (i / 4)
// + 4 hh + i % 4 (element i, lane half hh) of output column nw + 32 c + ln;
// each row is stored at its pair id's row of y.  Every pair of the layer
// belongs to exactly one tile row, so the down kernel writes all of y.
__device__ __forceinline__ void store_y_rows(float* y, int H, int nw, const int32_t* rpair, int rows,
                                             int lane, const f32x16 (&R)[4][4]) {
    const int ln = lane & 31, h4 = 4 * (lane >> 5);
    const int32_t* rp = rpair + h4;
    float* ybase = y + nw + ln;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int rc = mt * 32 + 8 * (i >> 2) + (i & 3);
            if (rc + h4 < rows) {
                float* yrow = ybase + static_cast<int64_t>(rp[rc]) * H;
#pragma unroll
                for (int c = 0; c < 4; ++c) __builtin_nontemporal_store(R[mt][c][i], yrow + 32 * c);
            }
        }
}

// Combine [FT-zh, Core method: a token's expert outputs merge into one sum]:
// out[t] = sum over j ascending of w[t, j] y[t k + j], fp32, 4 columns a thread.
typedef float f32x4 __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(256) combine_rows_kernel(const f32x4* __restrict__ y,
                                                           const float* __restrict__ w, int k,
                                                           uint32_t H4, uint32_t n4,
                                                           f32x4* __restrict__ out) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= n4) return;
    const uint32_t t = i / H4, c = i - t * H4;
    const f32x4* yr = y + static_cast<int64_t>(t) * k * H4 + c;
    const float* wt = w + static_cast<int64_t>(t) * k;
    f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < k; ++j) {
        const float wj = wt[j];
        const f32x4 v = __builtin_nontemporal_load(yr + static_cast<int64_t>(j) * H4);
        a.x = fmaf(wj, v.x, a.x);
        a.y = fmaf(wj, v.y, a.y);
        a.z = fmaf(wj, v.z, a.z);
        a.w = fmaf(wj, v.w, a.w);
    }
    out[i] = a;
}

moe355_status launch_combine(const float* y, const float* w, int T, int k, int H, float* out,
                             hipStream_t stream, const char* what) {
    const uint32_t H4 = static_cast<uint32_t>(H / 4);
    const uint32_t n4 = static_cast<uint32_t>(T) * H4;
    combine_rows_kernel<<<(n4 + 255) / 256, 256, 0, stream>>>(reinterpret_cast<const f32x4*>(y), w, k,
                                                              H4, n4, reinterpret_cast<f32x4*>(out));
    return check_launch(what);
}

// ---------------------------------------------------------------------------
// down: A = the tile's 128 rows of h (hi and lo); B = down rows nw + [0, 128)
// for wavefront w, nw = n0 + 128 w, as 4 column tiles; the y rows go to the
// pair-indexed array (a lane holds one output column of 16 rows per row tile,
// so each store instruction covers 128 contiguous bytes of 2 rows).
template <int FMT>
__global__ void __launch_bounds__(256) down_mfma(PrefillParams p) {
    constexpr int PD = DN_PD, OPS = 14;   // loads per stage per wavefront
    extern __shared__ uint4 smem[];
    uint8_t* ring = reinterpret_cast<uint8_t*>(smem);                  // [PD][DN_SLOT]
    int32_t* rpair = reinterpret_cast<int32_t*>(ring + PD * DN_SLOT);
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int H = p.H, I = p.I, Gd = I / 64, KS = I / BK;
    const int FX = (H + DN_COLS - 1) / DN_COLS;
    const uint32_t ring_lds = lds_addr(ring);
    const TileRange tr = tile_range(ld_const(p.n_tiles) * FX);
    for (int t = tr.begin; t < tr.end; t += tr.step) {
        const int y = t / FX;
        const int e = ld_const(p.tile_e + y), m0 = ld_const(p.tile_m0 + y);
        const int pbase = ld_const(p.offsets + e) + m0;
        const int rows = min(BM, ld_const(p.offsets + e + 1) - pbase);
        const void* W = uniform_ptr(p.W + static_cast<int64_t>(e) * p.S);
        const uint8_t* Wb = p.W + static_cast<int64_t>(e) * p.S;
        const int nw = (t - y * FX) * DN_COLS + 128 * wv;
        // The lane index is made opaque once per tile so that the compiler
        // recomputes lane-derived addresses here instead of hoisting dozens of
        // them out of the tile loop (they would spill, and every reload of a
        // spill waits for all memory operations in flight).
        int lane = tid & (WAVE - 1);
        asm volatile("" : "+v"(lane));
        const int ln = lane & 31, hh = lane >> 5;
        const bool live = nw < H;            // idle wavefronts of a small H compute on row 0
        const int nr = live ? nw : 0;
        const void* hb = uniform_ptr(p.h_hi + static_cast<int64_t>(pbase) * I);   // h rows are the bucket's pairs
        const void* lb = uniform_ptr(p.h_lo + static_cast<int64_t>(pbase) * I);
        __syncthreads();   // the previous tile is done with the LDS
        if (tid < BM) rpair[tid] = tid < rows ? p.perm[pbase + tid] : -1;   // pair id t k + j
        uint32_t aoff[4];   // rows past the bucket re-read its first row
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 8 * (4 * wv + j) + lane / 8, c = (lane % 8) ^ swz8(r);
            aoff[j] = static_cast<uint32_t>(r < rows ? r : 0) * static_cast<uint32_t>(2 * I) + c * 16;
        }
        uint32_t bq[4], bsc[2];
#pragma unroll
        for (int c = 0; c < 4; ++c) bq[c] = code_src(p.q_off[2], nr + 32 * c + ln, I, hh);
#pragma unroll
        for (int j = 0; j < 2; ++j) bsc[j] = scale_src(p.s_off[2], nr + 64 * j + lane, I);

        f32x16 R[4][4];   // [row tile][column tile]
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) R[i][c] = f32x16{};
        // Operands: a stage's weight codes and scale dwords, and the A fragments of
        // two MFMA steps [step][part hi / lo][row tile].
        struct WOps {
            uint4 q[4];
            uint32_t sc[4];
        };
        struct AOps {
            uint4 a[2][2][4];
        };
        // load i (of OPS) of stage kk into the slot at LDS address sl
        auto load_op = [&](int kk, uint32_t sl, int i) {
            if (i < 8) {
                const int j = i >> 1;
                dma16((i & 1) ? lb : hb, aoff[j] + kk * 128, sl + ((i & 1) ? DN_AL : DN_AH) + (4 * wv + j) * 1024);
            } else if (i < 12) {
                dma16(W, bq[i - 8] + code_step(kk), sl + DN_B + (4 * wv + i - 8) * 1024);
            } else {
                dma4(W, bsc[i - 12] + scale_step(kk), sl + DN_S + (2 * wv + i - 12) * 256);
            }
        };
        auto read_w = [&](const uint8_t* sp, int c, WOps& o) {
            o.q[c] = (reinterpret_cast<const uint4*>(sp + DN_B) + 4 * wv * 64 + lane)[c * 64];
            o.sc[c] = tile_scale(reinterpret_cast<const uint32_t*>(sp + DN_S), wv, c, ln);
        };
        // A fragment (step s0 + sx, part pt, row tile mt) into o.a[sx][pt][mt]
        auto read_a = [&](const uint8_t* sp, int s0, int i, AOps& o) {
            const int sx = i >> 3, pt = (i >> 2) & 1, mt = i & 3;
            o.a[sx][pt][mt] = a_operand(reinterpret_cast<const uint4*>(sp + (pt ? DN_AL : DN_AH)), mt, ln, hh, s0 + sx);
        };
        // The MFMAs of steps s0, s0 + 1 of stage kk: per step and column tile the
        // weight operand is dequantised (one group ahead) and used by the hi and
        // lo parts of every row tile; between the MFMAs, extra(j) issues reads
        // and loads.
        auto half = [&](auto NMTc, int kk, int s0, const WOps& w, const AOps& A, auto extra) {
            constexpr int NMT = decltype(NMTc)::value;
            uint4 b[2];
            b[0] = b_operand<FMT>(w.q[0], w.sc[0], kk, hh, s0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int g = 0; g < 8; ++g) {   // group g: step s0 + g / 4, column tile g % 4
#pragma unroll
                for (int m = 0; m < 2 * NMT; ++m) {
                    const int mt = m >> 1, pt = m & 1;
                    R[mt][g & 3] = mma<FMT>(A.a[g >> 2][pt][mt], b[g & 1], R[mt][g & 3]);
                    if (m == 0 && g + 1 < 8)
                        b[(g + 1) & 1] = b_operand<FMT>(w.q[(g + 1) & 3], w.sc[(g + 1) & 3], kk, hh, s0 + ((g + 1) >> 2));
                    extra(g * 2 * NMT + m);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        // Iteration kk: steps 0, 1 of stage kk (from X) while steps 2, 3 are read
        // into Y; the barrier (stage kk + 1 has landed, stage kk is read out);
        // steps 2, 3 (from Y) while stage kk + 1's weights and steps 0, 1 are read
        // into nw_ and X and the loads of stage kk + PD are issued.
        auto iter = [&](auto NMTc, int kk, int slot, const WOps& w, WOps& wn, AOps& X, AOps& Y) {
            constexpr int NMT = decltype(NMTc)::value;
            const uint8_t* sp = ring + slot * DN_SLOT;
            const int nslot = slot == PD - 1 ? 0 : slot + 1;
            const uint8_t* spn = ring + nslot * DN_SLOT;
            const uint32_t sl = ring_lds + slot * DN_SLOT;
            const int kl = min(kk + PD, KS - 1);
            // the 2 x 2 x NMT fragments of a half, in the order [step][part][row tile]
            auto frag = [&](int u) { return (u / (2 * NMT)) * 8 + ((u / NMT) & 1) * 4 + u % NMT; };
            half(NMTc, kk, 0, w, X, [&](int j) {
                if (j < 4 * NMT) read_a(sp, 2, frag(j), Y);
            });
            stage_barrier<OPS * (PD - 2)>();
            half(NMTc, kk, 2, w, Y, [&](int j) {
                if (j < 4) read_w(spn, j, wn);
                else if (j < 4 + 4 * NMT) read_a(spn, 0, frag(j - 4), X);
                if (j >= 2 && j - 2 < OPS) load_op(kl, sl, j - 2);
            });
        };
        auto kloop = [&](auto NMTc) {
            constexpr int NMT = decltype(NMTc)::value;
            WOps w0, w1;
            AOps X, Y;
#pragma unroll
            for (int s4 = 0; s4 < PD; ++s4)
#pragma unroll
                for (int i = 0; i < OPS; ++i) load_op(s4 < KS ? s4 : KS - 1, ring_lds + s4 * DN_SLOT, i);
            stage_barrier<OPS * (PD - 1)>();   // stage 0 has landed everywhere
#pragma unroll
            for (int c = 0; c < 4; ++c) read_w(ring, c, w0);
#pragma unroll
            for (int u = 0; u < 4 * NMT; ++u)
                read_a(ring, 0, (u / (2 * NMT)) * 8 + ((u / NMT) & 1) * 4 + u % NMT, X);
            int slot = 0;
#pragma nounroll
            for (int kk = 0; kk < KS; kk += 2) {   // KS is even
                iter(NMTc, kk, slot, w0, w1, X, Y);
                slot = slot == PD - 1 ? 0 : slot + 1;
                iter(NMTc, kk + 1, slot, w1, w0, X, Y);
                slot = slot == PD - 1 ? 0 : slot + 1;
            }
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");   // the repeated loads have landed
        };
        switch (__builtin_amdgcn_readfirstlane((rows + 31) / 32)) {
            case 1: kloop(std::integral_constant<int, 1>{}); break;
            case 2: kloop(std::integral_constant<int, 2>{}); break;
            case 3: kloop(std::integral_constant<int, 3>{}); break;
            default: kloop(std::integral_constant<int, 4>{}); break;
        }

        if (FMT == MOE355_W_INT4_G64) {
            for (int g0 = 0; g0 < Gd; g0 += 16) {
                const int gl = g0 + 8 * hh, BG = Gd;
                BiasRaw rb[4], ra[4];   // every load of the 16 groups first, then one wait
#pragma unroll
                for (int c = 0; c < 4; ++c) bias_b_load(Wb, p, 2, nr + 32 * c + ln, Gd, gl, rb[c]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const int r = mt * 32 + ln;
                    bias_a_load(p.hsum + static_cast<int64_t>(pbase + (r < rows ? r : 0)) * Gd, Gd, gl, ra[mt]);
                }
                uint4 bh[4], bl[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) bias_b_cvt(rb[c], BG, gl, &bh[c], &bl[c]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    uint4 xh, xl;
                    bias_a_cvt(ra[mt], BG, gl, &xh, &xl);
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        R[mt][c] = mma<FMT>(xh, bh[c], R[mt][c]);
                        R[mt][c] = mma<FMT>(xl, bh[c], R[mt][c]);
                        R[mt][c] = mma<FMT>(xh, bl[c], R[mt][c]);
                    }
                }
            }
        }

        if (live) store_y_rows(p.y, H, nw, rpair, rows, lane, R);
    }
}

// ---------------------------------------------------------------------------
// Native fp4 matrix-core path for MXFP4 experts: v_mfma_scale_f32_32x32x64_f8f6f4
// with the e2m1 weights (and their e8m0 block scales) as one operand and MX
// FP8 E4M3 activations (OCP Microscaling v1.0: 32 elements per e8m0 scale) as
// the other, so the products run on the fp8 x fp4 matrix-core rate.
//   x is quantised once per call (mx8_x_kernel): blocks of 32 along H.
//   gate/up: tile 128 pairs x 256 features, K = 128 per stage (two MFMAs of
//     K = 64); h = silu(g) * u leaves the accumulators as two MX terms
//     h1 = MX(h), h2 = MX(h - h1) per pair in blocks of 32 along I, so that a
//     rounding decision that differs between implementations in h's last bits
//     moves the sum h1 + h2 by at most one step of the second term.
//   down: tile 128 pairs x 512 outputs, K = 64 per stage, both terms of h
//     against the same weight operand; y rows and the combine as in the
//     f16/bf16 path.

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Shared exponent of an MX FP8 E4M3 block from its largest magnitude:
// floor(log2(amax)) - 8, clamped to e8m0's range; -127 for zero (and for amax
// below the normal range, whose floor(log2) is below -126).
__device__ __forceinline__ int mx_exponent(float amax) {
    const int ef = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFFu);
    const int e = ef - 127 - 8;
    return ef == 0 ? -127 : (e < -127 ? -127 : (e > 127 ? 127 : e));
}
// 2^-e for e in [-127, 119] (every block of finite bf16 or fp32 values), exact.
__device__ __forceinline__ float mx_inv_scale(int e) {
    return __uint_as_float(static_cast<uint32_t>(127 - e) << 23);
}
__device__ __forceinline__ float mx_scale(int e) {   // 2^e for e in [-127, 119], exact
    return e >= -126 ? __uint_as_float(static_cast<uint32_t>(127 + e) << 23)
                     : __uint_as_float(0x00400000u);   // 2^-127 (subnormal)
}

// FP8 E4M3 code of v (already divided by the block scale): round to nearest,
// ties to even, saturating at +-448; zero (of either sign) is code 0.  *q gets
// the code's value.  Done on the fp32 bits so the result is exact by construction.
__device__ __forceinline__ uint32_t e4m3_rne(float v, float* q) {
    const float a = fminf(__builtin_fabsf(v), 448.0f);
    uint32_t code;
    float mag;
    if (a < 0.015625f) {                           // below 2^-6: steps of 2^-9
        const float m = __builtin_rintf(a * 512.0f);   // 0 .. 8 (8 is 2^-6, code 0x08)
        code = static_cast<uint32_t>(m);
        mag = m * 0.001953125f;
    } else {                                       // keep 3 mantissa bits, nearest even
        const uint32_t b = __float_as_uint(a);
        const uint32_t r = (b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u;
        code = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);   // biased exponent - 127 + 7
        mag = __uint_as_float(r);
    }
    const bool neg = v < 0.0f && code != 0u;
    *q = neg ? -mag : mag;
    return code | (neg ? 0x80u : 0u);
}

// Four E4M3 codes of values already divided by their block scale, by gfx950's
// conversion (round to nearest, ties to even; checked against the rounding
// above on every bf16 pattern, tie neighbourhoods from 2^-16 to 2^9 and 2e6
// log-uniform draws: no difference except that a negative value that rounds
// to zero gets code 0x80, -0, which the down GEMM reads as zero).  Inputs are
// clamped to +-448 first, so the conversion never sees a value it would not
// saturate.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
    d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}
// The value of byte B of four E4M3 codes (exact).
template <int B>
__device__ __forceinline__ float e4m3_byte_value(uint32_t w) {
    return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(w), B);
}

// MX FP8 E4M3 copy of x: codes [T][H] and scale bytes [T][H / 32].  A thread
// takes 8 bf16 values (one 16-byte load); 4 neighbouring threads form a block.
__global__ void __launch_bounds__(256) mx8_x_kernel(const uint16_t* __restrict__ x, int64_t n8,
                                                    uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ scales) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (i < n8) v = reinterpret_cast<const uint4*>(x)[i];
    float f[8];
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = __uint_as_float(w4[j] << 16);
        f[2 * j + 1] = __uint_as_float(w4[j] & 0xFFFF0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, __builtin_fabsf(f[j]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, WAVE));
    amax = fmaxf(amax, __shfl_xor(amax, 2, WAVE));
    const int e = mx_exponent(amax);
    const float inv = mx_inv_scale(e);
    uint32_t c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float q;
        c[j] = e4m3_rne(f[j] * inv, &q);
    }
    if (i < n8) {
        reinterpret_cast<uint2*>(codes)[i] = make_uint2(c[0] | c[1] << 8 | c[2] << 16 | c[3] << 24,
                                                        c[4] | c[5] << 8 | c[6] << 16 | c[7] << 24);
        if ((i & 3) == 0) scales[i >> 2] = static_cast<uint8_t>(e + 127);
    }
}

// v_mfma_scale_f32_32x32x64_f8f6f4 operand layouts (measured on gfx950 with a
// one-wavefront check of random operands): lane l serves row (or column)
// l % 32 and half hf = l / 32 of the 64 inputs.
//   e2m1 operand: 16 bytes, inputs 32 hf + [0, 32), low nibble first;
//   E4M3 operand: 32 bytes, bytes 0-15 are inputs 16 hf + [0, 16) and bytes
//     16-31 inputs 32 + 16 hf + [0, 16);
//   scale: byte 0 of lane l's scale word is the e8m0 scale of inputs
//     32 hf + [0, 32) of its row, whichever lanes hold them.
__device__ __forceinline__ f32x16 mma_fp4_fp8(const uint4& w, uint32_t w_scale, const i32x8& x,
                                              uint32_t x_scale, f32x16 c) {
    const i32x8 a = {static_cast<int>(w.x), static_cast<int>(w.y), static_cast<int>(w.z),
                     static_cast<int>(w.w), 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, x, c, 4, 0, 0, static_cast<int>(w_scale),
                                                          0, static_cast<int>(x_scale));
}
// The same with the activation as the first operand (rows) and the weights as
// the second (columns).
__device__ __forceinline__ f32x16 mma_fp8_fp4(const i32x8& x, uint32_t x_scale, const uint4& w,
                                              uint32_t w_scale, f32x16 c) {
    const i32x8 b = {static_cast<int>(w.x), static_cast<int>(w.y), static_cast<int>(w.z),
                     static_cast<int>(w.w), 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, b, c, 0, 4, 0, static_cast<int>(x_scale),
                                                          0, static_cast<int>(w_scale));
}

struct MxParams {
    const uint8_t* xq;       // [T][H] MX FP8 E4M3 codes of x
    const uint8_t* xe;       // [T][H / 32] their scale bytes
    const int32_t* perm;
    const int32_t* offsets;
    const float* topk_w;
    const uint8_t* W;
    int64_t S;
    int64_t q_off[3], s_off[3];
    int T, k, H, I, E;
    const int32_t* tile_e;
    const int32_t* tile_m0;
    const int32_t* n_tiles;
    uint8_t* hq[2];          // [T*k][I] the two MX terms of h (rows in bucket order)
    uint8_t* he[2];          // [T*k][I / 32] their scale bytes
    float* y;                // [T*k][H] down outputs by pair id t k + j
};

// gate/up stage slot (K = 64): activation rows 128 x 64 bytes (16-byte chunk c of
// row r at slot c ^ swz4(r)); weights [wavefront][4 column tiles][64 lanes] x 16
// bytes in MFMA operand order; weight scale dwords [wavefront][2][64] (row
// 64 j + i of load j); activation scale dwords [wavefront][64] (row 32 w + i at
// i < 32).  A scale dword holds the e8m0 bytes of 128 inputs: stage kk uses
// bytes 2 (kk & 1) + {0, 1}.
constexpr int MG_A = 0, MG_W = 8192, MG_WS = 24576, MG_XS = 26624, MG_SLOT = 27648, MG_PD = 5;
constexpr int MG_K = 64;
// down stage slot (K = 64): two h terms of 128 rows x 64 bytes (chunk c of row r
// at slot c ^ swz4(r)); weights [wavefront][4][64] x 16 bytes; weight scale
// dwords [wavefront][2][64]; h scale dwords per term [wavefront][64].
constexpr int MD_A0 = 0, MD_A1 = 8192, MD_W = 16384, MD_WS = 32768, MD_HS = 34816,
              MD_SLOT = 36864, MD_PD = 4;
constexpr int MD_K = 64;

// One stage's MFMA operands of a lane: the weight codes of the 4 column tiles,
// the activations of the 4 row tiles, and the raw scale dwords.
struct MxOps {
    uint4 q[4];
    i32x8 x[4];
    uint32_t ws[4], xs[4];
};

// gate/up on the MX operands.  Per tile, stages of K = 64 flow through a ring of
// PD slots filled by direct loads: at the top of iteration kk every wavefront
// waits for stage kk + 1 and meets the others, after which stage kk's slot
// (already copied to registers) takes stage kk + PD; the 16 MFMAs of stage kk
// then run from registers while, between them, the next stage's operands are
// read from LDS into the other register set and the loads of stage kk + PD are
// issued.  The MFMA pipe so never waits on LDS, and the one barrier per stage
// finds the next stage already landed as long as the loads of PD - 2 stages
// cover the memory latency.  Past the last stage the loads repeat it (in
// bounds, never read), which keeps every wait count uniform; they drain before
// the next tile reuses the ring.
__global__ void __launch_bounds__(256) gate_up_mx(MxParams p) {
    constexpr int PD = MG_PD, OPS = 9;   // loads per stage per wavefront
    extern __shared__ uint4 smem[];
    uint8_t* ring = reinterpret_cast<uint8_t*>(smem);                  // [PD][MG_SLOT]
    int32_t* rtok = reinterpret_cast<int32_t*>(ring + PD * MG_SLOT);   // token of each tile row
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int H = p.H, I = p.I, KS = H / MG_K;
    const uint32_t ring_lds = lds_addr(ring);

    const int FX = (I + GU_FEAT - 1) / GU_FEAT;
    const TileRange tr = tile_range(ld_const(p.n_tiles) * FX);
    const void* xs = uniform_ptr(p.xq);
    const void* xes = uniform_ptr(p.xe);
    // The lane index is made opaque again for every tile (below), so that the
    // compiler recomputes lane-derived addresses per tile instead of hoisting
    // dozens of them out of the tile loop (they would spill, and a spill reload
    // waits for every memory operation in flight, the next tile's loads too).
    int lane = tid & (WAVE - 1), ln = 0, hh = 0;
    auto refresh_lane = [&]() {
        asm volatile("" : "+v"(lane));
        ln = lane & 31;
        hh = lane >> 5;
    };

    // A tile's load sources for this lane (the expert's blob, activation rows,
    // activation scale dwords, weight codes and scale dwords).  Setting them up
    // writes the tile's row tokens to LDS between two barriers.
    struct Src {
        const void* W;
        uint32_t aoff[2], xsoff, bq[4], bsc[2];
    };
    // this thread's pair of tile t (threads below BM; rows past the bucket
    // re-read its first row), loaded ahead of its use in setup
    auto tile_pair = [&](int t) {
        const int y = t / FX;
        const int e = ld_const(p.tile_e + y), m0 = ld_const(p.tile_m0 + y);
        const int pbase = ld_const(p.offsets + e) + m0;
        const int rows = min(BM, ld_const(p.offsets + e + 1) - pbase);
        return tid < BM ? p.perm[pbase + (tid < rows ? tid : 0)] : 0;
    };
    auto setup = [&](int t, Src& src, int pair) {
        const int y = t / FX;
        const int e = ld_const(p.tile_e + y);
        const int fw = (t - y * FX) * GU_FEAT + 64 * wv;
        const int fr = fw < I ? fw : 0;   // idle wavefronts of a small I compute on row 0
        src.W = uniform_ptr(p.W + static_cast<int64_t>(e) * p.S);
        __syncthreads();   // nobody reads the previous tokens any more
        if (tid < BM) rtok[tid] = pair / p.k;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 2; ++j) {   // 2 blocks of 16 rows x 4 chunks
            const int r = 16 * (2 * wv + j) + lane / 4, c = (lane % 4) ^ swz4(r);
            src.aoff[j] = static_cast<uint32_t>(rtok[r]) * static_cast<uint32_t>(H) + c * 16;
        }
        // activation scale dwords: row 32 wv + ln (both lane halves load it)
        src.xsoff = static_cast<uint32_t>(rtok[32 * wv + ln]) * static_cast<uint32_t>(H / 32);
#pragma unroll
        for (int c = 0; c < 4; ++c) src.bq[c] = code_src(p.q_off[c >> 1], fr + 32 * (c & 1) + ln, H, hh);
#pragma unroll
        for (int j = 0; j < 2; ++j) src.bsc[j] = scale_src(p.s_off[j], fr + lane, H);
    };
    // load i (of OPS) of stage kk into the slot at LDS address sl
    auto load_op = [&](const Src& src, int kk, uint32_t sl, int i) {
        if (i < 2) {
            dma16(xs, src.aoff[i] + kk * MG_K, sl + MG_A + (2 * wv + i) * 1024);
        } else if (i < 6) {
            dma16(src.W, src.bq[i - 2] + code_step(kk), sl + MG_W + (4 * wv + i - 2) * 1024);
        } else if (i < 8) {
            dma4(src.W, src.bsc[i - 6] + scale_step(kk), sl + MG_WS + (2 * wv + i - 6) * 256);
        } else {
            dma4(xes, src.xsoff + (kk >> 1) * 4, sl + MG_XS + wv * 256);
        }
    };
    // the first PD stages of a tile (the last stage again where KS < PD)
    auto prologue = [&](const Src& src) {
#pragma unroll
        for (int s = 0; s < PD; ++s)
#pragma unroll
            for (int i = 0; i < OPS; ++i) load_op(src, s < KS ? s : KS - 1, ring_lds + s * MG_SLOT, i);
    };
    // read piece i (of 16) of the stage in slot sp into o
    auto read_op = [&](const uint8_t* sp, int i, MxOps& o) {
        if (i < 4) {
            o.ws[i] = tile_scale(reinterpret_cast<const uint32_t*>(sp + MG_WS), wv, i, ln);
        } else if (i < 8) {
            o.xs[i - 4] = reinterpret_cast<const uint32_t*>(sp + MG_XS)[(i - 4) * 64 + ln];
        } else if (i < 12) {
            o.q[i - 8] = (reinterpret_cast<const uint4*>(sp + MG_W) + 4 * wv * 64 + lane)[(i - 8) * 64];
        } else {
            // inputs 16 hh + [0, 16) and 32 + 16 hh + [0, 16) of row tile i - 12
            const uint4* A = reinterpret_cast<const uint4*>(sp + MG_A);
            const int r = (i - 12) * 32 + ln;
            const uint4 u0 = A[r * 4 + (hh ^ swz4(r))];
            const uint4 u1 = A[r * 4 + ((2 + hh) ^ swz4(r))];
            o.x[i - 12] = i32x8{static_cast<int>(u0.x), static_cast<int>(u0.y), static_cast<int>(u0.z),
                                static_cast<int>(u0.w), static_cast<int>(u1.x), static_cast<int>(u1.y),
                                static_cast<int>(u1.z), static_cast<int>(u1.w)};
        }
    };

    Src src;
    if (tr.begin < tr.end) {
        refresh_lane();
        setup(tr.begin, src, tile_pair(tr.begin));
        prologue(src);
    }
    for (int t = tr.begin; t < tr.end; t += tr.step) {
        refresh_lane();
        // the next tile's pair ids: loaded now, used after this tile's K loop
        const int next_pair = t + tr.step < tr.end ? tile_pair(t + tr.step) : 0;
        const int y = t / FX;
        const int e = ld_const(p.tile_e + y), m0 = ld_const(p.tile_m0 + y);
        const int pbase = ld_const(p.offsets + e) + m0;
        const int rows = min(BM, ld_const(p.offsets + e + 1) - pbase);
        const int fw = (t - y * FX) * GU_FEAT + 64 * wv;
        const bool live = fw < I;
        // row tiles of 32 the MFMAs cover: a bucket's last tile is often short,
        // and its empty row tiles are skipped
        const int nmt = __builtin_amdgcn_readfirstlane((rows + 31) / 32);

        f32x16 R[4][4];   // [column tile][row tile]: features x tokens
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) R[c][i] = f32x16{};
        // iteration kk: MFMAs of stage kk from cur, reads of stage kk + 1 into nxt,
        // loads of stage kk + PD (the last stage again past the end)
        auto iter = [&](auto NMTc, int kk, int slot, const MxOps& cur, MxOps& nxt) {
            constexpr int NMT = decltype(NMTc)::value;
            stage_barrier<OPS * (PD - 2)>();   // stage kk + 1 has landed everywhere
            const int nslot = slot == PD - 1 ? 0 : slot + 1;
            const uint8_t* spn = ring + nslot * MG_SLOT;
            const uint32_t sl = ring_lds + slot * MG_SLOT;
            const int kl = min(kk + PD, KS - 1);
            const int sb = 8 * (2 * (kk & 1) + hh);   // this lane's scale byte
            uint32_t wsb[4], xsb[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) wsb[c] = (cur.ws[c] >> sb) & 0xFFu;
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) xsb[mt] = (cur.xs[mt] >> sb) & 0xFFu;
            __builtin_amdgcn_sched_barrier(0);
            // the reads go out with the first 8 MFMAs (done long before the next
            // barrier's wait for them), the loads with MFMAs 4 to 12
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int c = j >> 2, mt = j & 3;
                if (mt < NMT) R[c][mt] = mma_fp4_fp8(cur.q[c], wsb[c], cur.x[mt], xsb[mt], R[c][mt]);
#pragma unroll
                for (int i = 2 * j; i < 2 * j + 2; ++i)
                    if (i < 12 || (i < 16 && i - 12 < NMT)) read_op(spn, i, nxt);
                if (j >= 4 && j - 4 < OPS) load_op(src, kl, sl, j - 4);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // The tile's stages.  Its first PD stages were issued before the previous
        // tile's epilogue (or above, for the first tile); the wait for stage 0
        // also covers the memory operations issued in between (vector memory
        // operations of a wavefront complete in issue order).
        auto kloop = [&](auto NMTc) {
            MxOps o0, o1;
            stage_barrier<OPS * (PD - 1)>();   // stage 0 has landed everywhere
#pragma unroll
            for (int i = 0; i < 16; ++i) read_op(ring, i, o0);
            int slot = 0;
#pragma nounroll
            for (int kk = 0; kk < KS; kk += 2) {   // KS is even
                iter(NMTc, kk, slot, o0, o1);
                slot = slot == PD - 1 ? 0 : slot + 1;
                iter(NMTc, kk + 1, slot, o1, o0);
                slot = slot == PD - 1 ? 0 : slot + 1;
            }
            // the repeated loads have landed and every read of the ring is done
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        };
        switch (nmt) {
            case 1: kloop(std::integral_constant<int, 1>{}); break;
            case 2: kloop(std::integral_constant<int, 2>{}); break;
            case 3: kloop(std::integral_constant<int, 3>{}); break;
            default: kloop(std::integral_constant<int, 4>{}); break;
        }
        // the next tile's first stages load while this one's epilogue runs
        __builtin_amdgcn_sched_barrier(0);
        if (t + tr.step < tr.end) {
            setup(t + tr.step, src, next_pair);   // its first barrier: every wavefront is past the ring
            prologue(src);
        }
        __builtin_amdgcn_sched_barrier(0);

        mfma_drain();
        // h = silu(g) * u as two MX terms.  Lane (ln, hh) holds, for tile row
        // 32 mt + ln, features fw + 32 ft + 8 (i / 4) + 4 hh + i % 4 in R[ft][mt][i]
        // (g) and R[2 + ft][mt][i] (u): an MX block of 32 features is one column
        // tile, 16 values here and 16 in lane ln + 32 (the other half).
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int r = mt * 32 + ln;
            const bool keep = live && r < rows;
            const int64_t prow = static_cast<int64_t>(pbase + r);
#pragma unroll
            for (int ft = 0; ft < 2; ++ft) {
                float v[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float g = acc_read(R[ft][mt][i]), u = acc_read(R[2 + ft][mt][i]);
                    v[i] = silu(g) * u;
                }
                const int f0 = fw + 32 * ft;
#pragma unroll
                for (int term = 0; term < 2; ++term) {
                    float amax = 0.0f;
#pragma unroll
                    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, __builtin_fabsf(v[i]));
                    amax = max_with_partner(amax);
                    const int ex = mx_exponent(amax);
                    const float inv = mx_inv_scale(ex), sc = mx_scale(ex);
                    uint32_t cw[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        cw[j] = e4m3x4(v[4 * j] * inv, v[4 * j + 1] * inv, v[4 * j + 2] * inv,
                                       v[4 * j + 3] * inv);
                        // the residual (exact): the next term's input
                        v[4 * j] -= e4m3_byte_value<0>(cw[j]) * sc;
                        v[4 * j + 1] -= e4m3_byte_value<1>(cw[j]) * sc;
                        v[4 * j + 2] -= e4m3_byte_value<2>(cw[j]) * sc;
                        v[4 * j + 3] -= e4m3_byte_value<3>(cw[j]) * sc;
                    }
                    // lane half 0 holds features 8 j + 0..3 of the block, half 1
                    // 8 j + 4..7: trading j = 2, 3 (half 0) for j = 0, 1 (half 1)
                    // leaves each half 16 consecutive bytes, one store
                    const uint32_t r0 = half_partner(hh ? cw[0] : cw[2], hh);
                    const uint32_t r1 = half_partner(hh ? cw[1] : cw[3], hh);
                    if (keep) {
                        uint8_t* dst = p.hq[term] + prow * I + f0 + 16 * hh;
                        *reinterpret_cast<uint4*>(dst) = hh ? make_uint4(r0, cw[2], r1, cw[3])
                                                            : make_uint4(cw[0], r0, cw[1], r1);
                        if (hh == 0) p.he[term][prow * (I / 32) + f0 / 32] = static_cast<uint8_t>(ex + 127);
                    }
                }
            }
        }
    }
}

// down on the two MX terms of h: A = the tile's 128 rows of h (each term with
// its scale bytes); B = down rows nw + [0, 128) of wavefront w as 4 column tiles
// of e2m1 codes; the y rows go to the pair-indexed array as in down_mfma.
// Pipelined as gate_up_mx, with each K = 64 stage in two halves: the MFMAs of
// term 0 run while term 1's operands are read; then, past the stage's barrier
// (the next stage has landed, this one is read out), the MFMAs of term 1 run
// while the next stage's weights and term-0 operands are read and a later
// stage's loads are issued.
struct MxDnOps {   // a stage's weight codes and scales, one term's h operands
    uint4 q[4];
    uint32_t ws[4];
    i32x8 a[4];
    uint32_t hs[4];
};

__global__ void __launch_bounds__(256) down_mx(MxParams p) {
    constexpr int PD = MD_PD, OPS = 12;   // loads per stage per wavefront
    extern __shared__ uint4 smem[];
    uint8_t* ring = reinterpret_cast<uint8_t*>(smem);                  // [PD][MD_SLOT]
    int32_t* rpair = reinterpret_cast<int32_t*>(ring + PD * MD_SLOT);
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int H = p.H, I = p.I, KS = I / MD_K;
    const int FX = (H + DN_COLS - 1) / DN_COLS;
    const uint32_t ring_lds = lds_addr(ring);
    const TileRange tr = tile_range(ld_const(p.n_tiles) * FX);
    int lane = tid & (WAVE - 1), ln = 0, hh = 0;   // opaque per tile, as in gate_up_mx
    auto refresh_lane = [&]() {
        asm volatile("" : "+v"(lane));
        ln = lane & 31;
        hh = lane >> 5;
    };

    // A tile's load sources for this lane: both h terms with their scales, the
    // expert's blob with the down codes and scales.
    struct Src {
        const void *W, *hb0, *hb1, *hs0, *hs1;
        uint32_t aoff[2], hsoff, bq[4], bsc[2];
    };
    auto setup = [&](int t, Src& src) {
        const int y = t / FX;
        const int e = ld_const(p.tile_e + y), m0 = ld_const(p.tile_m0 + y);
        const int pbase = ld_const(p.offsets + e) + m0;
        const int rows = min(BM, ld_const(p.offsets + e + 1) - pbase);
        const int nw = (t - y * FX) * DN_COLS + 128 * wv;
        const int nr = nw < H ? nw : 0;   // idle wavefronts of a small H compute on row 0
        src.W = uniform_ptr(p.W + static_cast<int64_t>(e) * p.S);
        src.hb0 = uniform_ptr(p.hq[0] + static_cast<int64_t>(pbase) * I);
        src.hb1 = uniform_ptr(p.hq[1] + static_cast<int64_t>(pbase) * I);
        src.hs0 = uniform_ptr(p.he[0] + static_cast<int64_t>(pbase) * (I / 32));
        src.hs1 = uniform_ptr(p.he[1] + static_cast<int64_t>(pbase) * (I / 32));
#pragma unroll
        for (int j = 0; j < 2; ++j) {   // 2 blocks of 16 rows x 4 chunks; rows past the bucket re-read row 0
            const int r = 16 * (2 * wv + j) + lane / 4, c = (lane % 4) ^ swz4(r);
            src.aoff[j] = static_cast<uint32_t>(r < rows ? r : 0) * static_cast<uint32_t>(I) + c * 16;
        }
        const int srow = 32 * wv + ln;
        src.hsoff = static_cast<uint32_t>(srow < rows ? srow : 0) * static_cast<uint32_t>(I / 32);
#pragma unroll
        for (int c = 0; c < 4; ++c) src.bq[c] = code_src(p.q_off[2], nr + 32 * c + ln, I, hh);
#pragma unroll
        for (int j = 0; j < 2; ++j) src.bsc[j] = scale_src(p.s_off[2], nr + 64 * j + lane, I);
    };
    // load i (of OPS) of stage kk into the slot at LDS address sl
    auto load_op = [&](const Src& src, int kk, uint32_t sl, int i) {
        if (i < 4) {
            const int j = i & 1;
            dma16(i < 2 ? src.hb0 : src.hb1, src.aoff[j] + kk * MD_K,
                  sl + (i < 2 ? MD_A0 : MD_A1) + (2 * wv + j) * 1024);
        } else if (i < 8) {
            dma16(src.W, src.bq[i - 4] + code_step(kk), sl + MD_W + (4 * wv + i - 4) * 1024);
        } else if (i < 10) {
            dma4(src.W, src.bsc[i - 8] + scale_step(kk), sl + MD_WS + (2 * wv + i - 8) * 256);
        } else {
            dma4(i == 10 ? src.hs0 : src.hs1, src.hsoff + (kk >> 1) * 4,
                 sl + MD_HS + (i - 10) * 1024 + wv * 256);
        }
    };
    auto prologue = [&](const Src& src) {
#pragma unroll
        for (int s = 0; s < PD; ++s)
#pragma unroll
            for (int i = 0; i < OPS; ++i) load_op(src, s < KS ? s : KS - 1, ring_lds + s * MD_SLOT, i);
    };
    // term te's h operand of row tile mt, and its scale dword
    auto read_a = [&](const uint8_t* sp, int te, int mt, MxDnOps& o) {
        const uint4* A = reinterpret_cast<const uint4*>(sp + (te ? MD_A1 : MD_A0));
        const int r = mt * 32 + ln;
        const uint4 u0 = A[r * 4 + (hh ^ swz4(r))];         // inputs 16 hh + [0, 16)
        const uint4 u1 = A[r * 4 + ((2 + hh) ^ swz4(r))];   // 32 + 16 hh + [0, 16)
        o.a[mt] = i32x8{static_cast<int>(u0.x), static_cast<int>(u0.y), static_cast<int>(u0.z),
                        static_cast<int>(u0.w), static_cast<int>(u1.x), static_cast<int>(u1.y),
                        static_cast<int>(u1.z), static_cast<int>(u1.w)};
    };
    auto read_hs = [&](const uint8_t* sp, int te, int mt, MxDnOps& o) {
        o.hs[mt] = reinterpret_cast<const uint32_t*>(sp + MD_HS + te * 1024)[mt * 64 + ln];
    };
    auto read_w = [&](const uint8_t* sp, int c, MxDnOps& o) {
        o.q[c] = (reinterpret_cast<const uint4*>(sp + MD_W) + 4 * wv * 64 + lane)[c * 64];
        o.ws[c] = tile_scale(reinterpret_cast<const uint32_t*>(sp + MD_WS), wv, c, ln);
    };

    Src src;
    for (int t = tr.begin; t < tr.end; t += tr.step) {
        refresh_lane();
        const int y = t / FX;
        const int e = ld_const(p.tile_e + y), m0 = ld_const(p.tile_m0 + y);
        const int pbase = ld_const(p.offsets + e) + m0;
        const int rows = min(BM, ld_const(p.offsets + e + 1) - pbase);
        const int nw = (t - y * FX) * DN_COLS + 128 * wv;
        const bool live = nw < H;
        const int nmt = __builtin_amdgcn_readfirstlane((rows + 31) / 32);   // row tiles with rows
        __syncthreads();   // the previous tile is done with the ring and the pair ids
        setup(t, src);
        prologue(src);
        if (tid < BM) rpair[tid] = tid < rows ? p.perm[pbase + tid] : -1;   // pair id t k + j

        // The MFMAs take h as their first operand: a lane holds one output column
        // of 16 pairs per row tile, so each store instruction writes 128
        // contiguous bytes of 2 rows (whole cache lines; the transposed layout,
        // 16-byte runs of 32 rows per instruction, measured twice as slow).
        f32x16 R[4][4];   // [row tile][column tile]: pairs x outputs
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) R[i][c] = f32x16{};
        // iteration kk: term 0 from cur (with term 1 read into t1), the barrier,
        // term 1 (with stage kk + 1's weights and term 0 read into nxt and the
        // loads of stage kk + PD)
        auto iter = [&](auto NMTc, int kk, int slot, const MxDnOps& cur, MxDnOps& t1, MxDnOps& nxt) {
            constexpr int NMT = decltype(NMTc)::value;
            const uint8_t* sp = ring + slot * MD_SLOT;
            const int nslot = slot == PD - 1 ? 0 : slot + 1;
            const uint8_t* spn = ring + nslot * MD_SLOT;
            const uint32_t sl = ring_lds + slot * MD_SLOT;
            const int kl = min(kk + PD, KS - 1);
            const int sb = 8 * (2 * (kk & 1) + hh);
            uint32_t wsb[4], hsb[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) wsb[c] = (cur.ws[c] >> sb) & 0xFFu;
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) hsb[mt] = (cur.hs[mt] >> sb) & 0xFFu;
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 16; ++j) {   // term 0
                const int mt = j >> 2, c = j & 3;
                if (mt < NMT) R[mt][c] = mma_fp8_fp4(cur.a[mt], hsb[mt], cur.q[c], wsb[c], R[mt][c]);
                if (j < 2 * NMT) {
                    if (j & 1) read_hs(sp, 1, j >> 1, t1);
                    else read_a(sp, 1, j >> 1, t1);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            stage_barrier<OPS * (PD - 2)>();   // stage kk + 1 has landed; stage kk is read out
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) hsb[mt] = (t1.hs[mt] >> sb) & 0xFFu;
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 16; ++j) {   // term 1
                const int mt = j >> 2, c = j & 3;
                if (mt < NMT) R[mt][c] = mma_fp8_fp4(t1.a[mt], hsb[mt], cur.q[c], wsb[c], R[mt][c]);
                if (j < 4) {
                    read_w(spn, j, nxt);
                } else if (j < 4 + 2 * NMT) {
                    if (j & 1) read_hs(spn, 0, (j - 4) >> 1, nxt);
                    else read_a(spn, 0, (j - 4) >> 1, nxt);
                }
                if (j >= 2 && j - 2 < OPS) load_op(src, kl, sl, j - 2);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        auto kloop = [&](auto NMTc) {   // the tile's stages
            constexpr int NMT = decltype(NMTc)::value;
            MxDnOps o0, o1, ot;
            stage_barrier<OPS * (PD - 1)>();   // stage 0 has landed everywhere
#pragma unroll
            for (int c = 0; c < 4; ++c) read_w(ring, c, o0);
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) {
                read_a(ring, 0, mt, o0);
                read_hs(ring, 0, mt, o0);
            }
            int slot = 0;
#pragma nounroll
            for (int kk = 0; kk < KS; kk += 2) {   // KS is even
                iter(NMTc, kk, slot, o0, ot, o1);
                slot = slot == PD - 1 ? 0 : slot + 1;
                iter(NMTc, kk + 1, slot, o1, ot, o0);
                slot = slot == PD - 1 ? 0 : slot + 1;
            }
            // the repeated loads have landed and every read of the ring is done
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        };
        switch (nmt) {
            case 1: kloop(std::integral_constant<int, 1>{}); break;
            case 2: kloop(std::integral_constant<int, 2>{}); break;
            case 3: kloop(std::integral_constant<int, 3>{}); break;
            default: kloop(std::integral_constant<int, 4>{}); break;
        }
        // (a next tile's first loads issued here would wait behind these stores
        // in the wavefront's 63-entry memory counter: measured slower)
        mfma_drain();
        if (live) store_y_rows(p.y, H, nw, rpair, rows, lane, R);
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

// MX path workspace: the error word's 256 bytes, the tile plan and count, the
// MX copy of x and its scales, the two MX terms of h and their scales, the
// pair-indexed y rows.
size_t prefill_mx_ws_bytes(const moe355_layer_desc* d, int T) {
    const size_t tk = static_cast<size_t>(T) * d->top_k;
    const size_t th = static_cast<size_t>(T) * d->hidden;
    return 256 + align256(2 * static_cast<size_t>(max_tiles(T, d->top_k, d->n_experts)) * 4) + 256 +
           align256(th) + align256(th / 32) + 2 * align256(tk * d->inter) +
           2 * align256(tk * d->inter / 32) + align256(tk * d->hidden * sizeof(float));
}

size_t prefill_ws_bytes(const moe355_layer_desc* d, int T) {
    const size_t tk = static_cast<size_t>(T) * d->top_k;
    const size_t xb = d->wfmt == MOE355_W_INT4_G64
                          ? align256(static_cast<size_t>(T) * d->hidden * 2) +
                                align256(static_cast<size_t>(T) * (d->hidden / 64) * 4) +
                                align256(tk * (d->inter / 64) * 4)
                          : 0;
    // the error word's 256 bytes, h, the tile plan, the tile count, int4's x copy
    // and sums, the pair-indexed y rows
    return 256 + align256(tk * d->inter * sizeof(float)) +
           align256(2 * static_cast<size_t>(max_tiles(T, d->top_k, d->n_experts)) * sizeof(int32_t)) +
           256 + xb + align256(tk * d->hidden * sizeof(float));
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
    // the gate/up kernel addresses x rows by 32-bit byte offsets
    MOE355_REQUIRE(static_cast<int64_t>(T) * d->hidden * 2 <= 0xFFFFFFFFll, MOE355_ENOTSUP,
                   "expert_ffn_prefill: T*H=%lld beyond 2^31 activations", static_cast<long long>(T) * d->hidden);
    const size_t need = prefill_ws_bytes(d, T);
    MOE355_REQUIRE(ws && ws_bytes >= need, MOE355_ECAPACITY,
                   "expert_ffn_prefill: workspace %zu < %zu bytes", ws_bytes, need);
    ExpertLayout L;
    expert_layout(d, &L);
    const size_t tk = static_cast<size_t>(T) * d->top_k;
    const bool int4 = d->wfmt == MOE355_W_INT4_G64;
    PrefillParams p{};
    p.err = static_cast<uint32_t*>(ws);            // first 256 bytes: the error word
    uint8_t* wsb = static_cast<uint8_t*>(ws) + 256;
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
    const size_t off_x = off_tiles + align256(2 * static_cast<size_t>(mt) * 4) + 256;
    uint16_t* xf = reinterpret_cast<uint16_t*>(wsb + off_x);
    float* xsum = reinterpret_cast<float*>(wsb + off_x + align256(static_cast<size_t>(T) * d->hidden * 2));
    p.xf = xf;
    p.xsum = xsum;
    p.hsum = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(xsum) +
                                      align256(static_cast<size_t>(T) * (d->hidden / 64) * 4));
    const size_t xb = int4 ? align256(static_cast<size_t>(T) * d->hidden * 2) +
                                 align256(static_cast<size_t>(T) * (d->hidden / 64) * 4) +
                                 align256(tk * (d->inter / 64) * 4)
                           : 0;
    p.y = reinterpret_cast<float*>(wsb + off_x + xb);

    plan_kernel<<<1, 1024, 0, stream>>>(offsets, d->n_experts, tiles, tiles + mt,
                                        const_cast<int32_t*>(p.n_tiles), p.err);
    st = check_launch("expert_ffn_prefill plan");
    if (st) return st;
    const int blocks = prefill_blocks();
    if (int4) {
        const int64_t n8 = static_cast<int64_t>(T) * d->hidden / 8;
        x16_kernel<<<static_cast<unsigned>((n8 + 255) / 256), 256, 0, stream>>>(
            p.x, n8, d->hidden / 64, xf, xsum, p.err);
        st = check_launch("expert_ffn_prefill x16");
        if (st) return st;
    }
    const size_t lds_gu = GU_PD * GU_SLOT + BM * 4;
    const size_t lds_dn = DN_PD * DN_SLOT + BM * 4;
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
    st = check_launch("expert_ffn_prefill down");
    if (st) return st;
    return launch_combine(p.y, topk_w, T, d->top_k, d->hidden, out, stream, "expert_ffn_prefill combine");
}

extern "C" moe355_status moe355_quantize_mx(const void* x_bf16, int64_t rows, int32_t cols,
                                            uint8_t* codes, uint8_t* scales, hipStream_t stream) {
    MOE355_REQUIRE(rows >= 0 && cols > 0 && cols % 32 == 0, MOE355_EINVAL,
                   "quantize_mx: rows=%lld cols=%d (a positive multiple of 32)",
                   static_cast<long long>(rows), cols);
    if (rows == 0) return ok();
    MOE355_REQUIRE(x_bf16 && codes && scales, MOE355_EINVAL, "quantize_mx: null pointer");
    const int64_t n8 = rows * cols / 8;
    MOE355_REQUIRE((n8 + 255) / 256 <= 0x7FFFFFFFll, MOE355_ENOTSUP, "quantize_mx: too many values");
    mx8_x_kernel<<<static_cast<unsigned>((n8 + 255) / 256), 256, 0, stream>>>(
        static_cast<const uint16_t*>(x_bf16), n8, codes, scales);
    return check_launch("quantize_mx");
}

extern "C" moe355_status moe355_expert_ffn_prefill_mx(const moe355_layer_desc* d, const void* x_bf16,
                                                      int32_t T, const int32_t* topk_ids,
                                                      const float* topk_w, const uint8_t* layer_w,
                                                      const int32_t* perm, const int32_t* offsets,
                                                      float* out, void* ws, size_t ws_bytes,
                                                      hipStream_t stream) {
    (void)topk_ids;
    moe355_status st = check_desc(d);
    if (st) return st;
    MOE355_REQUIRE(d->wfmt == MOE355_W_MXFP4, MOE355_ENOTSUP,
                   "expert_ffn_prefill_mx: MXFP4 experts only (wfmt=%d)", d->wfmt);
    MOE355_REQUIRE(T >= 0 && static_cast<int64_t>(T) * d->top_k < (1ll << 28), MOE355_EINVAL,
                   "expert_ffn_prefill_mx: T=%d", T);
    if (T == 0) return ok();
    MOE355_REQUIRE(x_bf16 && topk_w && layer_w && perm && offsets && out, MOE355_EINVAL,
                   "expert_ffn_prefill_mx: null pointer");
    MOE355_REQUIRE(d->hidden % 256 == 0 && d->inter % 128 == 0 && d->n_experts <= 1024 &&
                       d->hidden <= 16384 && d->inter <= 16384,
                   MOE355_ENOTSUP, "expert_ffn_prefill_mx: H=%d (multiple of 256), I=%d (of 128), E=%d",
                   d->hidden, d->inter, d->n_experts);
    // x rows and h rows are addressed by 32-bit byte offsets
    MOE355_REQUIRE(static_cast<int64_t>(T) * d->hidden <= 0xFFFFFFFFll &&
                       static_cast<int64_t>(T) * d->top_k * d->inter <= 0xFFFFFFFFll,
                   MOE355_ENOTSUP, "expert_ffn_prefill_mx: T*H or T*k*I beyond 2^32 bytes");
    const size_t need = prefill_mx_ws_bytes(d, T);
    MOE355_REQUIRE(ws && ws_bytes >= need, MOE355_ECAPACITY,
                   "expert_ffn_prefill_mx: workspace %zu < %zu bytes", ws_bytes, need);
    ExpertLayout L;
    expert_layout(d, &L);
    const size_t tk = static_cast<size_t>(T) * d->top_k, th = static_cast<size_t>(T) * d->hidden;
    const int mt = max_tiles(T, d->top_k, d->n_experts);
    uint8_t* at = static_cast<uint8_t*>(ws);
    uint32_t* err = reinterpret_cast<uint32_t*>(at);
    at += 256;
    int32_t* tiles = reinterpret_cast<int32_t*>(at);
    at += align256(2 * static_cast<size_t>(mt) * 4);
    int32_t* n_tiles = reinterpret_cast<int32_t*>(at);
    at += 256;
    MxParams p{};
    uint8_t* xq = at;
    at += align256(th);
    uint8_t* xe = at;
    at += align256(th / 32);
    for (int term = 0; term < 2; ++term) {
        p.hq[term] = at;
        at += align256(tk * d->inter);
    }
    for (int term = 0; term < 2; ++term) {
        p.he[term] = at;
        at += align256(tk * d->inter / 32);
    }
    p.y = reinterpret_cast<float*>(at);
    p.xq = xq;
    p.xe = xe;
    p.perm = perm;
    p.offsets = offsets;
    p.topk_w = topk_w;
    p.W = layer_w;
    p.S = L.bytes;
    for (int m = 0; m < 3; ++m) {
        p.q_off[m] = L.q_off[m];
        p.s_off[m] = L.s_off[m];
    }
    p.T = T;
    p.k = d->top_k;
    p.H = d->hidden;
    p.I = d->inter;
    p.E = d->n_experts;
    p.tile_e = tiles;
    p.tile_m0 = tiles + mt;
    p.n_tiles = n_tiles;

    plan_kernel<<<1, 1024, 0, stream>>>(offsets, d->n_experts, tiles, tiles + mt, n_tiles, err);
    st = check_launch("expert_ffn_prefill_mx plan");
    if (st) return st;
    const int64_t n8 = static_cast<int64_t>(th / 8);
    mx8_x_kernel<<<static_cast<unsigned>((n8 + 255) / 256), 256, 0, stream>>>(
        static_cast<const uint16_t*>(x_bf16), n8, xq, xe);
    st = check_launch("expert_ffn_prefill_mx quantise x");
    if (st) return st;
    const size_t lds_gu = MG_PD * MG_SLOT + BM * 4;
    const size_t lds_dn = MD_PD * MD_SLOT + BM * 4;
    static bool granted = false;
    if (!granted) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(gate_up_mx),
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                static_cast<int>(lds_gu)) != hipSuccess ||
            hipFuncSetAttribute(reinterpret_cast<const void*>(down_mx),
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                static_cast<int>(lds_dn)) != hipSuccess)
            return fail(MOE355_EHIP, "expert_ffn_prefill_mx: LDS %zu / %zu bytes refused", lds_gu, lds_dn);
        granted = true;
    }
    const int blocks = prefill_blocks();
    gate_up_mx<<<blocks, 256, lds_gu, stream>>>(p);
    st = check_launch("expert_ffn_prefill_mx gate_up");
    if (st) return st;
    down_mx<<<blocks, 256, lds_dn, stream>>>(p);
    st = check_launch("expert_ffn_prefill_mx down");
    if (st) return st;
    return launch_combine(p.y, topk_w, T, d->top_k, d->hidden, out, stream,
                          "expert_ffn_prefill_mx combine");
}
