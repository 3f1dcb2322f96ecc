// Internal helpers shared by the libmoe355 translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe355.h"

namespace moe355 {

// ---- host-side status -------------------------------------------------------
moe355_status fail(moe355_status s, const char* fmt, ...);
moe355_status check_launch(const char* what);
inline moe355_status ok() { return MOE355_OK; }

#define MOE355_REQUIRE(cond, code, ...) \
    do { if (!(cond)) return ::moe355::fail((code), __VA_ARGS__); } while (0)

// Bytes of one expert blob and the offsets of its tensors (canonical layout).
struct ExpertLayout {
    int64_t bytes = 0;
    // per matrix m (0 gate, 1 up, 2 down): packed codes, then scales (s or e), then biases
    int64_t q_off[3] = {0, 0, 0};
    int64_t s_off[3] = {0, 0, 0};
    int64_t b_off[3] = {0, 0, 0};
};
bool expert_layout(const moe355_layer_desc* d, ExpertLayout* L);
moe355_status check_desc(const moe355_layer_desc* d);
moe355_status check_cache(const moe355_cache* c);
moe355_status check_out(const moe355_classify_out* o, bool full, int n_ids);

// Routing of a call's tokens folded into the cache bookkeeping kernel.
struct RouteArgs {
    const float* logits;   // [T, E]
    int T, k, kind, n_group, topk_group;
    float scale;
    int32_t* ids_out;      // [T, k]
    float* w_out;          // [T, k]
};
// What one bookkeeping launch does.
enum ClassifyMode {
    CLASSIFY_FULL = 0,    // route?, dedup, hit/miss, victims, slot update, plan with fills
    CLASSIFY_DEDUP = 1,   // dedup and plan only, no cache
    CLASSIFY_PLAN = 2,    // route?, dedup, hit/miss and a plan reading misses from the pool
    CLASSIFY_EVICT = 3,   // hit stamps, victims, slot update and fill lists for a planned call
};
// The bookkeeping call's parameter block (classify_dev.h), checked and filled,
// and its launch as one workgroup.
struct ClassifyParams;
moe355_status classify_setup(const moe355_cache* c, int32_t layer, const int64_t* tick_dev,
                             int64_t tick, const int32_t* ids, int32_t n_ids,
                             const moe355_evict_policy* p, moe355_classify_out* out,
                             const RouteArgs* route, ClassifyMode mode, ClassifyParams* cp);
moe355_status classify_launch(const ClassifyParams& cp, hipStream_t stream);
moe355_status classify_call(const moe355_cache* c, int32_t layer, const int64_t* tick_dev,
                            int64_t tick, const int32_t* ids, int32_t n_ids,
                            const moe355_evict_policy* p, moe355_classify_out* out,
                            const RouteArgs* route, ClassifyMode mode, hipStream_t stream);
moe355_status fill_call(const moe355_cache* c, const uint8_t* pool, int32_t layer,
                        const moe355_classify_out* out, int32_t max_fill, hipStream_t stream);
// The whole decode layer call (bookkeeping and FFN with fill-through) as one
// launch when the call is small enough; *launched tells whether it was.
moe355_status decode_layer_small(const moe355_layer_desc* d, const moe355_cache* c,
                                 const uint8_t* pool, int32_t layer, const ClassifyParams& cp,
                                 const void* x_bf16, int32_t T, const int32_t* topk_ids,
                                 const float* topk_w, const moe355_classify_out* lists,
                                 const moe355_evict_policy* pol, float* out, void* ws,
                                 size_t ws_bytes, hipStream_t stream, bool* launched,
                                 uint32_t* err = nullptr);
// err: where the kernels record device-side failures (default: the workspace's
// error word at MOE355_DECODE_ERR_BYTE).
moe355_status decode_ffn(const moe355_layer_desc* d, const void* x_bf16, int32_t T,
                         const int32_t* topk_ids, const float* topk_w, const moe355_cache* cache,
                         const uint8_t* pool, int32_t layer, const moe355_classify_out* exp,
                         bool fill_through, float* out, void* ws, size_t ws_bytes,
                         hipStream_t stream, uint32_t* err = nullptr);
size_t decode_ws_bytes(const moe355_layer_desc* d, int T);

// ---- device helpers ---------------------------------------------------------
constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Order-preserving map of a float to uint32 (-0.0 folded onto +0.0 first).
__device__ __forceinline__ uint32_t f32_order_key(float v) {
    uint32_t u = __float_as_uint(v + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <typename T>
__device__ __forceinline__ T wave_xor(T v, int mask) {
    return __shfl_xor(v, mask, WAVE);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint64_t o = __shfl_xor(v, m, WAVE);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
    return v;
}

// 16 bytes written through to the device coherence point by two device-scope
// 8-byte stores (compiler-visible stores, so the hazard that a store's data
// registers must not be overwritten right after issue is handled for them).
__device__ __forceinline__ void st_dev16(void* q, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    uint64_t* w = static_cast<uint64_t*>(q);
    __hip_atomic_store(w, static_cast<uint64_t>(a) | static_cast<uint64_t>(b) << 32, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(w + 1, static_cast<uint64_t>(c) | static_cast<uint64_t>(d) << 32, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Minimum / maximum over the 64 lanes by DPP row shifts and row broadcasts (an
// inclusive scan; lane 63 ends with the result), without the LDS crossbar.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(~0u, v, 0x111, 0xf, 0xf, false)));  // row_shr:1
    v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(~0u, v, 0x112, 0xf, 0xf, false)));  // row_shr:2
    v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(~0u, v, 0x114, 0xf, 0xf, false)));  // row_shr:4
    v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(~0u, v, 0x118, 0xf, 0xf, false)));  // row_shr:8
    v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(~0u, v, 0x142, 0xa, 0xf, false)));  // row_bcast:15
    v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(~0u, v, 0x143, 0xc, 0xf, false)));  // row_bcast:31
    return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false)));
    return __builtin_amdgcn_readlane(v, 63);
}

// Sum over the 64 lanes by DPP row shifts and row broadcasts (an inclusive
// scan; lane 63 ends with the total), without the LDS crossbar.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                 ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_sum_dpp_f32(float v) {
    v += dpp_f32<0x111, 0xf>(v);   // row_shr:1
    v += dpp_f32<0x112, 0xf>(v);   // row_shr:2
    v += dpp_f32<0x114, 0xf>(v);   // row_shr:4
    v += dpp_f32<0x118, 0xf>(v);   // row_shr:8
    v += dpp_f32<0x142, 0xa>(v);   // row_bcast:15
    v += dpp_f32<0x143, 0xc>(v);   // row_bcast:31
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Error-word bits (include/moe355.h): a bounded wait gave up; an int4-path
// activation or intermediate fell outside f16's finite range.
constexpr uint32_t ERR_WAIT = 1u;
constexpr uint32_t ERR_F16_RANGE = 2u;

// Largest bf16 magnitude (as packed 16-bit pairs) of the 8 bf16 values in v,
// folded into acc: one mask and one packed 16-bit maximum per dword.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2_t bf16_mag_max(uint4 v, u16x2_t acc) {
    auto mag = [](uint32_t w) { return __builtin_bit_cast(u16x2_t, w & 0x7FFF7FFFu); };
    const u16x2_t a = __builtin_elementwise_max(mag(v.x), mag(v.y));
    const u16x2_t b = __builtin_elementwise_max(mag(v.z), mag(v.w));
    return __builtin_elementwise_max(acc, __builtin_elementwise_max(a, b));
}
// Whether a bf16 magnitude from bf16_mag_max lies beyond f16's finite range
// (|x| >= 65536 once in bf16; 0x4780 is 65536, 0x477F = 65280 still fits), or is
// inf or NaN.
__device__ __forceinline__ bool bf16_mag_beyond_f16(u16x2_t m) {
    return m.x >= 0x4780u || m.y >= 0x4780u;
}
// f16 rounding to nearest overflows from 65520 on.
__device__ __forceinline__ bool beyond_f16(float v) { return !(__builtin_fabsf(v) < 65520.0f); }

// Sum over aligned segments of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float segment_sum_f32(float v, int width) {
    for (int m = width >> 1; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
    return v;
}

}  // namespace moe355
