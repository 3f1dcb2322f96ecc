// GPU producer of the synthetic expert pool: the same bytes as
// workloads/experts.py (SplitMix64 counter generator, canonical blob layout),
// written straight into device memory so multi-gigabyte pools need no host copy.
// Input generation only.
#include <hip/hip_runtime.h>
#include <stdint.h>

// Every float step below must round exactly as the NumPy generator does: no
// fused multiply-adds.
#pragma clang fp contract(off)

namespace {

constexpr uint64_t GAMMA = 0x9E3779B97F4A7C15ull;

__device__ __host__ inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ inline uint64_t word(uint64_t base, uint64_t g, uint64_t region, uint64_t j) {
    const uint64_t ctr = (g << 36) | (region << 32) | j;
    return mix64(base + (ctr + 1) * GAMMA);
}

__device__ inline uint16_t bf16_rne(float f) {
    uint32_t b = __float_as_uint(f);
    return static_cast<uint16_t>((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

__device__ inline float uniform24(uint64_t w) {
    return __fmul_rn(static_cast<float>(static_cast<uint32_t>(w >> 40)), 5.9604644775390625e-08f);
}

struct Geo {
    int64_t S;
    int64_t q_off[3], s_off[3], b_off[3];
    int64_t nq[3];   // packed bytes per matrix
    int64_t ng[3];   // scale entries per matrix (int4: per 64, mx: per 32)
    int wfmt;
};

__global__ void synth_kernel(uint8_t* __restrict__ dst, int64_t g0, Geo geo, uint64_t base) {
    const int64_t g = g0 + blockIdx.y;
    uint8_t* blob = dst + static_cast<int64_t>(blockIdx.y) * geo.S;
    for (int m = 0; m < 3; ++m) {
        const int64_t nw = geo.nq[m] / 8;
        const int rq = geo.wfmt == 0 ? 3 * m : 2 * m;
        uint64_t* q = reinterpret_cast<uint64_t*>(blob + geo.q_off[m]);
        for (int64_t j = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; j < nw;
             j += static_cast<int64_t>(gridDim.x) * blockDim.x)
            q[j] = word(base, g, rq, j);
        if (geo.wfmt == 0) {
            uint16_t* s = reinterpret_cast<uint16_t*>(blob + geo.s_off[m]);
            uint16_t* b = reinterpret_cast<uint16_t*>(blob + geo.b_off[m]);
            for (int64_t j = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
                 j < geo.ng[m]; j += static_cast<int64_t>(gridDim.x) * blockDim.x) {
                const float us = uniform24(word(base, g, 3 * m + 1, j));
                const float sf = __fadd_rn(0.005f, __fmul_rn(0.015f, us));
                const uint16_t sb = bf16_rne(sf);
                const float ub = uniform24(word(base, g, 3 * m + 2, j));
                const float v = __fmul_rn(-8.0f, ub);
                const float bf = __fmul_rn(v, __uint_as_float(static_cast<uint32_t>(sb) << 16));
                s[j] = sb;
                b[j] = bf16_rne(bf);
            }
        } else {
            uint64_t* e = reinterpret_cast<uint64_t*>(blob + geo.s_off[m]);
            for (int64_t j = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
                 j < geo.ng[m] / 8; j += static_cast<int64_t>(gridDim.x) * blockDim.x) {
                const uint64_t w = word(base, g, 2 * m + 1, j);
                e[j] = (w & 0x0303030303030303ull) + 0x7676767676767676ull;  // 118 + (byte & 3)
            }
        }
    }
}

}  // namespace

// Fill `count` experts starting at global expert g0 (= layer * E + e) into dst
// ([count * S] bytes).  wfmt: 0 int4 g64, 1 MXFP4.  Returns 0 or a hipError_t.
extern "C" int synth_fill_experts(uint8_t* dst, int64_t g0, int64_t count, int wfmt, int H, int I,
                                  uint64_t seed, hipStream_t stream) {
    if (count <= 0) return 0;
    Geo geo{};
    geo.wfmt = wfmt;
    const int64_t dims[3][2] = {{I, H}, {I, H}, {H, I}};
    int64_t off = 0;
    for (int m = 0; m < 3; ++m) {
        const int64_t out = dims[m][0], in = dims[m][1];
        geo.q_off[m] = off;
        geo.nq[m] = out * in / 2;
        off += geo.nq[m];
        if (wfmt == 0) {
            geo.ng[m] = out * in / 64;
            geo.s_off[m] = off;
            off += 2 * geo.ng[m];
            geo.b_off[m] = off;
            off += 2 * geo.ng[m];
        } else {
            geo.ng[m] = out * in / 32;
            geo.s_off[m] = off;
            off += geo.ng[m];
        }
    }
    geo.S = off;
    const uint64_t base = mix64((seed + 1) * GAMMA);
    for (int64_t c0 = 0; c0 < count; c0 += 65535) {
        const int64_t n = count - c0 < 65535 ? count - c0 : 65535;
        dim3 grid(64, static_cast<unsigned>(n));
        synth_kernel<<<grid, 256, 0, stream>>>(dst + c0 * geo.S, g0 + c0, geo, base);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return static_cast<int>(e);
    }
    return 0;
}
