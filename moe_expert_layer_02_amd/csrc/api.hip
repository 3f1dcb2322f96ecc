// Host side of the C ABI: status reporting, descriptor checks, the canonical
// expert layout and workspace sizes.
#include <stdarg.h>
#include <stdio.h>

#include "internal.h"

namespace moe355 {

static thread_local char g_last_error[512] = "";

moe355_status fail(moe355_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

moe355_status check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE355_EHIP, "%s: %s", what, hipGetErrorString(e));
    return MOE355_OK;
}

// One expert: for gate [I,H], up [I,H], down [H,I]: q [out, in/2] then, for
// int4, s and b bf16 [out, in/64]; for MXFP4, e uint8 [out, in/32].
bool expert_layout(const moe355_layer_desc* d, ExpertLayout* L) {
    if (!d || d->hidden <= 0 || d->inter <= 0) return false;
    const int64_t H = d->hidden, I = d->inter;
    const int64_t dims[3][2] = {{I, H}, {I, H}, {H, I}};
    int64_t off = 0;
    for (int m = 0; m < 3; ++m) {
        const int64_t out = dims[m][0], in = dims[m][1];
        L->q_off[m] = off;
        off += out * in / 2;
        if (d->wfmt == MOE355_W_INT4_G64) {
            if (in % 64) return false;
            L->s_off[m] = off;
            off += 2 * (out * in / 64);
            L->b_off[m] = off;
            off += 2 * (out * in / 64);
        } else if (d->wfmt == MOE355_W_MXFP4) {
            if (in % 32) return false;
            L->s_off[m] = off;
            off += out * in / 32;
            L->b_off[m] = off;
        } else {
            return false;
        }
    }
    L->bytes = off;
    return true;
}

moe355_status check_desc(const moe355_layer_desc* d) {
    MOE355_REQUIRE(d, MOE355_EINVAL, "null layer descriptor");
    MOE355_REQUIRE(d->hidden > 0 && d->inter > 0 && d->n_experts > 0, MOE355_EINVAL,
                   "descriptor: H=%d I=%d E=%d", d->hidden, d->inter, d->n_experts);
    MOE355_REQUIRE(d->top_k >= 1 && d->top_k <= d->n_experts, MOE355_EINVAL, "descriptor: k=%d",
                   d->top_k);
    MOE355_REQUIRE(d->route == MOE355_ROUTE_SOFTMAX_TOPK || d->route == MOE355_ROUTE_SIGMOID_GROUP,
                   MOE355_EINVAL, "descriptor: route=%d", d->route);
    MOE355_REQUIRE(d->wfmt == MOE355_W_INT4_G64 || d->wfmt == MOE355_W_MXFP4, MOE355_EINVAL,
                   "descriptor: wfmt=%d", d->wfmt);
    if (d->route == MOE355_ROUTE_SIGMOID_GROUP)
        MOE355_REQUIRE(d->n_group >= 1 && d->topk_group >= 1 && d->topk_group <= d->n_group,
                       MOE355_EINVAL, "descriptor: n_group=%d topk_group=%d", d->n_group,
                       d->topk_group);
    MOE355_REQUIRE(d->hidden % 64 == 0 && d->inter % 64 == 0, MOE355_ENOTSUP,
                   "descriptor: H=%d and I=%d must be multiples of 64", d->hidden, d->inter);
    return MOE355_OK;
}

size_t permute_ws_bytes(int E, int T, int k);
size_t prefill_ws_bytes(const moe355_layer_desc* d, int T);
size_t prefill_mx_ws_bytes(const moe355_layer_desc* d, int T);
size_t decode_ws_bytes(const moe355_layer_desc* d, int T);

}  // namespace moe355

using namespace moe355;

extern "C" const char* moe355_status_string(moe355_status s) {
    switch (s) {
        case MOE355_OK: return "ok";
        case MOE355_EINVAL: return "invalid argument";
        case MOE355_EHIP: return "HIP error";
        case MOE355_ENOTSUP: return "unsupported shape or format";
        case MOE355_ECAPACITY: return "buffer too small";
        default: return "unknown status";
    }
}

extern "C" const char* moe355_last_error(void) { return g_last_error; }

#ifndef MOE355_SRC_SHA
#define MOE355_SRC_SHA "unknown"
#endif
// "libmoe355 <version> gfx950 src:<first 16 hex digits of the sources' sha256>"
extern "C" const char* moe355_version(void) { return "libmoe355 0.2 gfx950 src:" MOE355_SRC_SHA; }

extern "C" int64_t moe355_expert_bytes(const moe355_layer_desc* d) {
    ExpertLayout L;
    if (check_desc(d) != MOE355_OK || !expert_layout(d, &L)) return 0;
    return L.bytes;
}

extern "C" size_t moe355_workspace_bytes(const moe355_layer_desc* d, int32_t T, int32_t mode) {
    if (check_desc(d) != MOE355_OK || T < 0) return 0;
    switch (mode) {
        case MOE355_MODE_DECODE: return decode_ws_bytes(d, T);
        case MOE355_MODE_PREFILL: return prefill_ws_bytes(d, T);
        case MOE355_MODE_PERMUTE: return permute_ws_bytes(d->n_experts, T, d->top_k);
        case MOE355_MODE_PREFILL_MX: return prefill_mx_ws_bytes(d, T);
        default: return 0;
    }
}
