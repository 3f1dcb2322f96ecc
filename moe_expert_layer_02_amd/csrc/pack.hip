// Canonical -> device layout of expert blobs (a rearrangement of bytes only).
//
// Device layout: every region (codes, scales, biases) of each matrix is cut into
// blocks of 16 output rows x 128 inputs; a code block holds 16-byte chunk j of
// row r at (16 j + r) * 16, a scale/bias block holds row r's 4 bytes at 4 r.
#include <algorithm>

#include "internal.h"

namespace moe355 {
namespace {

// One thread per 16-byte code chunk of one matrix of every blob.
__global__ void pack_codes_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                  int64_t n_blobs, int64_t S, int64_t q_off, int rows, int in) {
    const int64_t chunks = static_cast<int64_t>(rows) * (in / 32);   // 16-byte chunks per matrix
    const int64_t total = n_blobs * chunks;
    const int kcs = in / 128;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t blob = i / chunks, o = i - blob * chunks;   // output chunk o
        const int64_t blk = o >> 6;
        const int w = static_cast<int>(o & 63), j = w >> 4, r = w & 15;
        const int64_t rt = blk / kcs, kc = blk - rt * kcs;
        const int64_t row = rt * 16 + r;
        const uint8_t* s = src + blob * S + q_off + row * (in / 2) + kc * 64 + j * 16;
        uint8_t* d = dst + blob * S + q_off + o * 16;
        *reinterpret_cast<uint4*>(d) = *reinterpret_cast<const uint4*>(s);
    }
}

// One thread per 4-byte word of one scale or bias region of every blob.
__global__ void pack_words_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                  int64_t n_blobs, int64_t S, int64_t off, int rows, int in) {
    const int64_t words = static_cast<int64_t>(rows) * (in / 128);
    const int64_t total = n_blobs * words;
    const int kcs = in / 128;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t blob = i / words, o = i - blob * words;
        const int64_t blk = o >> 4;
        const int r = static_cast<int>(o & 15);
        const int64_t rt = blk / kcs, kc = blk - rt * kcs;
        const int64_t row = rt * 16 + r;
        // a row of the region holds in/32 bytes (in/64 bf16, or in/32 e8m0)
        const uint8_t* s = src + blob * S + off + row * (in / 32) + kc * 4;
        uint8_t* d = dst + blob * S + off + o * 4;
        *reinterpret_cast<uint32_t*>(d) = *reinterpret_cast<const uint32_t*>(s);
    }
}

}  // namespace
}  // namespace moe355

using namespace moe355;

extern "C" moe355_status moe355_pack_experts(const moe355_layer_desc* d, const uint8_t* src,
                                             uint8_t* dst, int64_t n, hipStream_t stream) {
    moe355_status st = check_desc(d);
    if (st) return st;
    MOE355_REQUIRE(n >= 0, MOE355_EINVAL, "pack_experts: n=%lld", static_cast<long long>(n));
    if (n == 0) return ok();
    MOE355_REQUIRE(src && dst, MOE355_EINVAL, "pack_experts: null pointer");
    MOE355_REQUIRE(d->hidden % 128 == 0 && d->inter % 128 == 0, MOE355_ENOTSUP,
                   "pack_experts: H=%d and I=%d must be multiples of 128", d->hidden, d->inter);
    ExpertLayout L;
    MOE355_REQUIRE(expert_layout(d, &L), MOE355_EINVAL, "pack_experts: bad layout");
    const int64_t S = L.bytes;
    MOE355_REQUIRE(src + n * S <= dst || dst + n * S <= src, MOE355_EINVAL,
                   "pack_experts: src and dst overlap");
    const int dims[3][2] = {{d->inter, d->hidden}, {d->inter, d->hidden}, {d->hidden, d->inter}};
    const bool int4 = d->wfmt == MOE355_W_INT4_G64;
    for (int m = 0; m < 3; ++m) {
        const int rows = dims[m][0], in = dims[m][1];
        const int64_t chunks = n * rows * (in / 32);
        const unsigned gc = static_cast<unsigned>(std::min<int64_t>((chunks + 255) / 256, 65536));
        pack_codes_kernel<<<gc, 256, 0, stream>>>(src, dst, n, S, L.q_off[m], rows, in);
        const int64_t words = n * rows * (in / 128);
        const unsigned gw = static_cast<unsigned>(std::min<int64_t>((words + 255) / 256, 65536));
        pack_words_kernel<<<gw, 256, 0, stream>>>(src, dst, n, S, L.s_off[m], rows, in);
        if (int4) pack_words_kernel<<<gw, 256, 0, stream>>>(src, dst, n, S, L.b_off[m], rows, in);
        st = check_launch("pack_experts");
        if (st) return st;
    }
    return ok();
}
