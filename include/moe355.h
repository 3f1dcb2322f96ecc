/*
 * libmoe355 -- one MoE layer's forward pass on an AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every pointer argument named *device* is device memory owned by the
 * caller; the library allocates nothing on these paths and never synchronises
 * the host.  Every call is asynchronous on the given HIP stream and returns
 * after validating its arguments and enqueueing its kernels.  Shapes are fixed
 * per call; how many entries of a list are valid is reported in device memory
 * (the "counts" arrays), so a whole decode step can be enqueued without the
 * host reading anything back.
 *
 * Errors: a call returns MOE355_OK (0) or a negative status.  Argument,
 * shape, dtype and capacity problems are found on the host before anything is
 * enqueued, and nothing is launched then.  A failed launch returns
 * MOE355_EHIP.  moe355_last_error() gives a one-line description of the
 * most recent failure on the calling host thread.
 *
 * Sources (cited by page title and section):
 *   [FT-zh]  "FreeToken: Efficient Edge-Native MoE Serving with Bandwidth-Adaptive
 *            Execution", Chinese digest -- Core method, Method steps, Technical novelty.
 *   [FT-en]  the same paper's simplified English reader -- System Architecture,
 *            Semantic-Aware Expert Caching, Elastic Memory Management, Figure 2.
 *   [Edge0]  "The other half of the memory wall: serving a 35B MoE model from SSD
 *            with trained route prediction" (translation) -- section 2 (MoE routing,
 *            Quantization), section 3.1 (Problem, Executor paths, Math contract).
 */
#ifndef MOE355_H
#define MOE355_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe355_status;
#define MOE355_OK          0
#define MOE355_EINVAL     (-1)   /* bad pointer, size or parameter            */
#define MOE355_EHIP       (-2)   /* a HIP launch or runtime call failed        */
#define MOE355_ENOTSUP    (-3)   /* shape or format this build does not handle */
#define MOE355_ECAPACITY  (-4)   /* a caller buffer (list, workspace) too small */

/* Static text for a status code. */
const char* moe355_status_string(moe355_status s);
/* Description of the latest failure on this host thread ("" if none). */
const char* moe355_last_error(void);
/* Library version string: "libmoe355 <version> gfx950 src:<hash>", where <hash>
 * is the first 16 hex digits of the sha256 of the sources the library was
 * built from (so a loaded binary can be matched to its source tree). */
const char* moe355_version(void);

/*
 * Error words.  Some failures can only be seen on the device while a call runs;
 * they are recorded in a 32-bit word of the call's workspace, which the caller
 * reads after the call has completed:
 *   decode (moe355_expert_ffn_decode, moe355_decode_layer): the word at byte
 *     MOE355_DECODE_ERR_BYTE of the workspace, sticky (never cleared by the
 *     library: clear it with the rest of the workspace's first 65536 bytes);
 *   prefill (moe355_expert_ffn_prefill): the word at byte MOE355_PREFILL_ERR_BYTE,
 *     cleared by each call with T > 0 before its kernels run.
 * A set bit means the outputs of the call that set it are not valid:
 *   MOE355_ERR_WAIT      a bounded in-kernel wait gave up (one-launch decode calls);
 *   MOE355_ERR_F16_RANGE int4 weights only: an activation x (|x| > 65504 as a bf16
 *                        value, inf or NaN) or an intermediate h = silu(gate x) * (up x)
 *                        (times the routing weight inside the one-launch decode
 *                        calls; |h| >= 65520) lies outside f16's finite range.  The
 *                        int4 path runs its products on f16 operands; inside that
 *                        range they are exact, except that |x| < 2^-14 keeps only
 *                        the multiples of 2^-24 (an absolute error below 2^-24 per
 *                        element).  MXFP4 weights run on bf16 operands and have no
 *                        such limit.
 */
#define MOE355_DECODE_ERR_BYTE   4608
#define MOE355_PREFILL_ERR_BYTE  0
#define MOE355_ERR_WAIT          1u
#define MOE355_ERR_F16_RANGE     2u

/* Routing families [Edge0, section 2 "MoE routing"]. */
#define MOE355_ROUTE_SOFTMAX_TOPK   0
#define MOE355_ROUTE_SIGMOID_GROUP  1

/* Expert weight formats. */
#define MOE355_W_INT4_G64   0  /* int4 affine, group 64 along the input [Edge0, section 2 "Quantization"] */
#define MOE355_W_MXFP4      1  /* OCP MX v1.0: e2m1 elements, e8m0 scale per 32 along the input */

/*
 * One MoE layer's shape and routing (the model description the Edge0 page
 * calls MoESpec, section 3 Figure 1).  n_group / topk_group / route_scale are
 * read only for MOE355_ROUTE_SIGMOID_GROUP.
 */
typedef struct {
    int32_t hidden;      /* H */
    int32_t inter;       /* I, expert intermediate size */
    int32_t n_experts;   /* E */
    int32_t top_k;       /* k */
    int32_t route;       /* MOE355_ROUTE_* */
    int32_t n_group;
    int32_t topk_group;
    float   route_scale;
    int32_t wfmt;        /* MOE355_W_* */
} moe355_layer_desc;

/*
 * Bytes of one expert, S.  One expert is a contiguous blob with, for gate
 * [I,H], up [I,H] and down [H,I] in that order, a code region, a scale region
 * and (int4 only) a bias region.  In the canonical layout ([Edge0, section 2]
 * affine int4 in groups of 64, OCP MX for MXFP4) int4 stores q uint8
 * [out, in/2] (element 2c in the low nibble of byte c), s bf16 [out, in/64]
 * and b bf16 [out, in/64] (weight = s*q + b); MXFP4 stores q uint8 [out, in/2]
 * (e2m1 codes, same nibble order) and e uint8 [out, in/32] (scale 2^(e-127)).
 * Returns 0 for an invalid descriptor.
 */
int64_t moe355_expert_bytes(const moe355_layer_desc* d);

/*
 * The device layout, read by every expert FFN call and kept in the pool, the
 * cache slots and the prefill layer buffer: the same regions at the same
 * offsets, each cut into blocks of 16 output rows x 128 inputs, block
 * (rt, kc) at index rt * (in/128) + kc.
 *   code block, 1024 bytes: the 16-byte chunk j (inputs 32j..32j+31 of the
 *     block) of row r sits at byte (16 j + r) * 16;
 *   scale (and bias) block, 64 bytes: row r's 4 bytes at 4 r, the canonical
 *     bytes that cover the block's 128 inputs (two bf16 group values for
 *     int4, four e8m0 exponents for MXFP4).
 * A wavefront reads a block with one contiguous 1 KB load and its scales with
 * one 64-byte load (the canonical layout needs one memory request per row).
 * Requires hidden and inter to be multiples of 128.
 *
 * moe355_pack_experts: n experts from the canonical layout at src to the
 * device layout at dst (device arrays of n * S bytes that must not overlap).
 * Asynchronous on `stream`.  Errors: MOE355_EINVAL for a bad descriptor, null
 * pointers or n < 0; MOE355_ENOTSUP when hidden or inter is not a multiple of
 * 128.
 */
moe355_status moe355_pack_experts(const moe355_layer_desc* d, const uint8_t* src, uint8_t* dst,
                                  int64_t n, hipStream_t stream);

/*
 * The HBM expert cache [FT-zh, Core method: N slots shared by every MoE layer,
 * each holding the complete tensors of one (layer, expert); the pool stays the
 * source of truth].  All arrays are device memory owned by the caller.
 *   slot_table [n_layers*n_experts] int32: slot of (l, e) or -1.
 *   slot_owner [n_slots] int32: l*E+e held by the slot, or -1.
 *   slot_ts    [n_slots] int64: tick of the last router selection, 0 = never used.
 *   slot_data  [n_slots * slot_bytes].
 * A fresh cache is table = -1, owner = -1, ts = 0.
 */
typedef struct {
    int32_t  n_slots;
    int32_t  n_layers;
    int32_t  n_experts;
    int64_t  slot_bytes;
    int32_t* slot_table;
    int32_t* slot_owner;
    int64_t* slot_ts;
    uint8_t* slot_data;
} moe355_cache;

/*
 * Miss handling [FT-zh, Core method: q* = m * B_P / B_H; FT-en, Semantic-Aware
 * Expert Caching: rounded to nearest].  q = min(m, floor((2*q_num*m + q_den) /
 * (2*q_den))); q_num = q_den = 1 is pure fill.  K is the number of LRU victims
 * one scan returns [FT-en, Elastic Memory Management]; at most min(q, K) misses
 * are filled, the rest are computed in place from the pool.
 */
typedef struct {
    int32_t K;
    int32_t q_num;
    int32_t q_den;
} moe355_evict_policy;

/*
 * Per-call lists, each of `capacity` int32 device entries, plus
 * counts[6] = {n_uniq, n_hit, n_miss, n_fill, n_inplace, n_victims}.
 * uniq, hit_expert, miss, fill_expert and inplace hold expert ids in ascending
 * order; hit_slot / fill_slot pair with hit_expert / fill_expert; victims are
 * slots in ascending (ts, slot) order.  Entries past the counts are unspecified.
 *
 * plan [capacity][4] int32 and pairs [pair_capacity] int32 describe the call for
 * the expert FFN, one row per distinct expert uniq[u]:
 *   plan[u] = {slot holding the expert after the call or -1 (read from the pool),
 *              1 if this call fills that slot else 0,
 *              first index into pairs, number of pairs};
 * pairs lists the routed (token, slot) pairs t*k + j grouped by u.
 * pair_capacity must be >= the call's number of routed ids.
 */
typedef struct {
    int32_t* uniq;
    int32_t* hit_expert;
    int32_t* hit_slot;
    int32_t* miss;
    int32_t* fill_expert;
    int32_t* fill_slot;
    int32_t* inplace;
    int32_t* victims;
    int32_t* counts;
    int32_t  capacity;
    int32_t* plan;
    int32_t* pairs;
    int32_t  pair_capacity;
} moe355_classify_out;

/*
 * Router projection: logits[t, e] = sum_h x[t, h] * w_router[e, h], fp32
 * accumulation.  The routing families of [Edge0, section 2 "MoE routing"] score
 * per-expert logits of each token; no page spells out how the logits are formed,
 * and this call forms them with the plain linear router x . W_r^T.
 * x: device bf16 [T, H]; w_router: device fp32 [E, H]; logits: device fp32 [T, E].
 * Errors: MOE355_EINVAL for a bad descriptor, null pointers or T < 0.
 */
moe355_status moe355_router_logits(const moe355_layer_desc* d, const void* x_bf16,
                                   const float* w_router, int32_t T, float* logits,
                                   hipStream_t stream);

/*
 * Routing [Edge0, section 2 "MoE routing"].
 *   softmax-top-k: the k largest fp32 logits (ties to the lower expert id),
 *     w_j = exp(l_j - l_max) / sum over the kept of exp(l - l_max).
 *   sigmoid-group: s = sigmoid(l) in fp64; groups are n_group blocks of E/n_group
 *     consecutive experts ranked by the sum of their two largest s (fp64, ties to
 *     the lower group); the best topk_group groups are kept; the k largest logits
 *     inside them are chosen (ties to the lower id); w = s / sum(s) * route_scale.
 * ids are written in descending score order.
 * logits: device fp32 [T, E]; topk_ids: device int32 [T, k]; topk_w: device fp32 [T, k].
 * Limits: E <= 512, k <= 32 and k <= E; for sigmoid-group E/n_group must hold
 * at least 2 experts and the group size must split evenly over lanes
 * (E/n_group a power of two, or a multiple of ceil(E/64)).
 */
moe355_status moe355_route(const moe355_layer_desc* d, const float* logits, int32_t T,
                           int32_t* topk_ids, float* topk_w, hipStream_t stream);

/*
 * Dedup only: uniq = sorted distinct ids of ids[0..n_ids), counts[0] = their
 * number; the other counts are set to 0.  Used when no cache is present
 * (whole layer resident).  out->capacity must be >= min(n_ids, E).
 */
moe355_status moe355_dedup(const int32_t* ids, int32_t n_ids, int32_t n_experts,
                           moe355_classify_out* out, hipStream_t stream);

/*
 * One layer call's cache bookkeeping, as one single-workgroup kernel
 * [FT-zh, Core method and Method steps; FT-en, Elastic Memory Management]:
 * dedup the n_ids routed ids of `layer`; split them into hits (slot_table >= 0)
 * and misses; stamp hits with `tick`; compute q; scan every slot's timestamp once
 * and take the K smallest (ts, slot) among slots with ts < tick as victims;
 * for i < min(q, n_victims): evict victim i's owner (its table entry -> -1), map
 * miss i to victim i, set owner and ts = tick.  Remaining misses go to `inplace`.
 * The caller must use a tick larger than every earlier one (e.g. step*L + l + 1).
 * Limits: n_slots <= 16384, n_experts <= 1024, n_ids <= 1024, 0 < tick < 2^31,
 * out->capacity >= max(min(n_ids, E), K).  (The device keeps timestamps as 32-bit
 * values: calls that take the tick from device memory, tick_base below, must keep
 * it under 2^32, which the host cannot check.)
 */
moe355_status moe355_classify_evict(const moe355_cache* c, int32_t layer, int64_t tick,
                                    const int32_t* ids, int32_t n_ids,
                                    const moe355_evict_policy* p, moe355_classify_out* out,
                                    hipStream_t stream);

/*
 * Batch copy of the filled experts [FT-zh, Core method: batch copy inside the
 * graph]: for i < counts[3], S bytes from pool + (layer*E + fill_expert[i]) * S
 * to slot_data + fill_slot[i] * S.  pool: device [n_layers * E * S].
 * max_fill bounds counts[3] (use the policy's K).
 */
moe355_status moe355_cache_fill(const moe355_cache* c, const uint8_t* pool, int32_t layer,
                                const moe355_classify_out* out, int32_t max_fill,
                                hipStream_t stream);

/*
 * Elastic rebuild at a safe point [FT-en, Elastic Memory Management: the slot
 * count follows the memory budget and excess slots are evicted without a
 * restart]: `to` (to->n_slots slots, same n_layers / n_experts / slot_bytes)
 * receives the to->n_slots occupied slots of `from` that are last in
 * (ts, slot) order, packed into slots 0.. in ascending old-slot order with
 * their timestamps and bytes; remaining slots of `to` are empty.  `from` is
 * read only.  No byte of `to`'s four arrays may overlap any byte of `from`'s
 * (table n_layers*n_experts*4, owner n_slots*4, ts n_slots*8, data
 * n_slots*slot_bytes bytes): MOE355_EINVAL otherwise.
 */
moe355_status moe355_cache_rebuild(const moe355_cache* from, moe355_cache* to,
                                   hipStream_t stream);

/*
 * Prefill bucketing.  No page defines this call: it groups a prefill batch's
 * routed pairs by expert so that the whole-layer path of [Edge0, section 3.1
 * "Executor paths"] runs each expert once over its token bucket.  It is a stable
 * sort of the T*k pairs p = t*k + j by expert id.
 * perm: device int32 [T*k]; offsets: device int32 [E+1] (offsets[e] = first
 * position of expert e, offsets[E] = T*k).  ws: device scratch of
 * moe355_workspace_bytes(d, T, MOE355_MODE_PERMUTE) bytes.  Errors: MOE355_EINVAL
 * for a bad descriptor, null pointers or ids; MOE355_ECAPACITY for a short
 * workspace.
 */
moe355_status moe355_permute(const moe355_layer_desc* d, const int32_t* topk_ids, int32_t T,
                             int32_t* perm, int32_t* offsets, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/*
 * Decode expert FFN with the combine fused [Edge0, section 3.1 "Math contract":
 * down(silu(gate(x)) * up(x)); FT-zh, Core method: partial sums merge exactly]:
 *   out[t] = sum_j topk_w[t, j] * down_e(silu(gate_e(x_t)) * up_e(x_t)),  e = topk_ids[t, j].
 * The distinct experts are read from uniq / counts[0] of `exp` (filled by
 * moe355_classify_evict or moe355_dedup); each expert's bytes are read once per
 * call, from its cache slot when cache != NULL and slot_table[layer*E+e] >= 0,
 * else from pool + (layer*E + e) * S (pool = one layer's buffer with layer = 0
 * for a whole-layer call).  x: device bf16 [T, H]; out: device fp32 [T, H];
 * ws: device scratch of moe355_workspace_bytes(d, T, MOE355_MODE_DECODE) bytes
 * (calls sharing one workspace must not overlap).  Its first 65536 bytes hold
 * the call's synchronisation counters and flags: zero them once when the
 * workspace is allocated; every call leaves them zero, except the sticky error
 * word at byte MOE355_DECODE_ERR_BYTE (see "Error words" above).  exp->plan and
 * exp->pairs (written by moe355_classify_evict or moe355_dedup) are required.
 * Kernels: a small call (T <= 16, H in {1024, 2048, 4096}, distinct experts x
 * I/16 <= the device's compute units, T*k*I*4 <= 32 KiB) runs as one launch in
 * which the down blocks wait for the gate/up blocks and each pair of them owns
 * 16 output rows of all experts (two fp32 additions per element onto zero,
 * which give the same sum in either order: the output is deterministic).
 * Otherwise two
 * kernels: gate/up (which also zeroes out), then down with the combine as fp32
 * atomic additions, so the order of a token's k additions is not fixed.
 * Limits: T*k <= 256; H and I in {128, 256, 512, 1024, 2048, 4096}.
 */
moe355_status moe355_expert_ffn_decode(const moe355_layer_desc* d, const void* x_bf16,
                                       int32_t T, const int32_t* topk_ids, const float* topk_w,
                                       const moe355_cache* cache, const uint8_t* pool,
                                       int32_t layer, const moe355_classify_out* exp,
                                       float* out, void* ws, size_t ws_bytes,
                                       hipStream_t stream);

/*
 * One whole decode layer call [FT-zh, Method steps: per layer a
 * single device kernel routes, deduplicates, classifies, splits the misses and
 * picks the LRU victims; the GPU computes G = H u F while F is copied into its
 * slots; everything replays inside one captured graph with no host
 * involvement]: route T tokens from `logits`, run the bookkeeping of
 * moe355_classify_evict, then the expert FFN of moe355_expert_ffn_decode with
 * the combine.  The experts filled in this call are read from the pool and
 * their bytes are written to their victim slots by the FFN itself (the same end
 * state as moe355_cache_fill, one fewer pass over those bytes).
 *   tick = *tick_base + tick_add when tick_base (device int64) is non-null,
 *   else tick_add; it must exceed every earlier tick.
 * logits: device fp32 [T, E]; x: device bf16 [T, H]; topk_ids / topk_w: device
 * [T, k] outputs; lists: the call's classify lists (capacity >= max(min(T*k, E),
 * K)); out: device fp32 [T, H]; ws as for moe355_expert_ffn_decode.
 * Kernels: a small call (the small-call rule of moe355_expert_ffn_decode, plus a
 * cache of at most 2048 slots, E <= 256, T*k <= 128 and K <= 128; every
 * one-token Qwen-like call) runs as ONE launch whose first workgroup does the
 * routing and bookkeeping and publishes the plan to the FFN workgroups;
 * otherwise the bookkeeping kernel runs first and the expert FFN after it.
 * Limits: 1 <= T*k <= 256, plus those of the two calls; tick < 2^32.
 */
moe355_status moe355_decode_layer(const moe355_layer_desc* d, const moe355_cache* c,
                                  const uint8_t* pool, int32_t layer, const int64_t* tick_base,
                                  int64_t tick_add, const float* logits, const void* x_bf16,
                                  int32_t T, const moe355_evict_policy* p, int32_t* topk_ids,
                                  float* topk_w, moe355_classify_out* lists, float* out, void* ws,
                                  size_t ws_bytes, hipStream_t stream);

/*
 * moe355_decode_layer without a workspace, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments and results as moe355_decode_layer, minus
 * ws / ws_bytes: the call's synchronisation words and h live in a fixed scratch
 * array inside the library, one per GPU, held until the process ends
 * (64 KiB + 4 MiB: T*k*I <= 2^20, which every shape the decode kernels take
 * meets -- T*k <= 256, I <= 4096; else MOE355_ECAPACITY before anything is
 * enqueued).  Nothing is allocated: the first call on a device looks the
 * array's address up and clears its synchronisation words with a kernel on
 * `stream`; every call leaves them zero again.
 * err_word: device uint32 owned by the caller, which the call ORs its error
 * bits into (see "Error words"; the same bits the workspace's error word
 * would get).  Every call on one GPU shares that GPU's scratch: calls that
 * overlap on one GPU (other streams, other host threads) race and must be
 * ordered by the caller.
 */
moe355_status moe355_decode_layer_static(const moe355_layer_desc* d, const moe355_cache* c,
                                         const uint8_t* pool, int32_t layer,
                                         const int64_t* tick_base, int64_t tick_add,
                                         const float* logits, const void* x_bf16, int32_t T,
                                         const moe355_evict_policy* p, int32_t* topk_ids,
                                         float* topk_w, moe355_classify_out* lists, float* out,
                                         uint32_t* err_word, hipStream_t stream);

/*
 * The same layer call with the cache bookkeeping off the critical path
 * [FT-zh, Core method: VRAM only changes speed, never results; FT-zh, Method
 * steps: the filled experts are batch-copied into their victim slots].  Three
 * calls replace moe355_decode_layer:
 *   1. moe355_route_plan on the compute stream: route T tokens from `logits`,
 *      deduplicate, classify hits and misses against the slot table (read only)
 *      and write lists->uniq / hit / miss, counts[0..2] (counts[3..5] = 0), the
 *      pairs and a plan in which hits read their slots and misses the pool.
 *   2. moe355_expert_ffn_decode on the compute stream with `lists` and the cache.
 *   3. moe355_evict_fill on a second stream, ordered after call 1: stamps the
 *      hits with the tick, selects the K LRU victims, splits the misses by q,
 *      updates slot_table / slot_owner / slot_ts, writes lists->fill / inplace /
 *      victims and counts[3..5], and copies the filled experts from the pool
 *      into their victim slots.  It never touches the slots this call reads.
 * The next call that reads the slot table (any layer) must be ordered after
 * call 3.  The results equal moe355_decode_layer's; the filled experts' bytes
 * are read twice (once by the FFN, once by the copy).
 * Arguments as for moe355_decode_layer; T*k <= 256.
 */
moe355_status moe355_route_plan(const moe355_layer_desc* d, const moe355_cache* c, int32_t layer,
                                const float* logits, int32_t T, int32_t* topk_ids, float* topk_w,
                                moe355_classify_out* lists, hipStream_t stream);

moe355_status moe355_evict_fill(const moe355_layer_desc* d, const moe355_cache* c,
                                const uint8_t* pool, int32_t layer, const int64_t* tick_base,
                                int64_t tick_add, const int32_t* topk_ids, int32_t T,
                                const moe355_evict_policy* p, moe355_classify_out* lists,
                                hipStream_t stream);

/*
 * Prefill expert FFN: a grouped GEMM over each expert's token bucket (from
 * moe355_permute) on the matrix cores, with the whole layer resident
 * [Edge0, section 3.1 "Executor paths": the whole-layer path loads all experts
 * of a layer for prefill; FT-zh, Method steps].  Same result as the decode
 * call.  layer_w: device [E * S].  out: device fp32 [T, H].
 * ws: moe355_workspace_bytes(d, T, MOE355_MODE_PREFILL) bytes, whose word at
 * MOE355_PREFILL_ERR_BYTE is the call's error word (see "Error words").
 * Limits: H a multiple of 256 up to 8192, I a multiple of 128 up to 2048,
 * E <= 1024, T*H < 2^31.
 */
moe355_status moe355_expert_ffn_prefill(const moe355_layer_desc* d, const void* x_bf16,
                                        int32_t T, const int32_t* topk_ids, const float* topk_w,
                                        const uint8_t* layer_w, const int32_t* perm,
                                        const int32_t* offsets, float* out, void* ws,
                                        size_t ws_bytes, hipStream_t stream);

/*
 * MX FP8 E4M3 quantisation of bf16 activations (OCP Microscaling Formats v1.0;
 * the activation operand of moe355_expert_ffn_prefill_mx): each row of x is cut
 * into blocks of 32; a block's shared exponent is e = floor(log2(max |x|)) - 8
 * (clamped to [-127, 127]; -127 for a zero block), stored as the byte e + 127;
 * each element x / 2^e is rounded to the nearest E4M3 value (ties to even),
 * saturating at +-448, and a zero element is stored as 0x00.
 * x: device bf16 [rows, cols]; codes: device uint8 [rows, cols]; scales: device
 * uint8 [rows, cols / 32].  Errors: MOE355_EINVAL for rows < 0, cols not a
 * positive multiple of 32, or null pointers when rows > 0.
 */
moe355_status moe355_quantize_mx(const void* x_bf16, int64_t rows, int32_t cols, uint8_t* codes,
                                 uint8_t* scales, hipStream_t stream);

/*
 * Prefill expert FFN for MXFP4 experts on the native fp4 matrix cores
 * (v_mfma_scale_f32_32x32x64_f8f6f4): the e2m1 weights with their e8m0 block
 * scales against MX FP8 E4M3 activations (the pages' MXFP4 models are the
 * DeepSeek-V4-Flash rows of [FT-zh, Results]).  Same call shape as moe355_expert_ffn_prefill, but
 * a different result: x is quantised as moe355_quantize_mx does (per token,
 * blocks of 32 along H), and h = silu(gate x) * (up x) is carried into the down
 * projection as two MX FP8 terms per routed pair (blocks of 32 along I):
 * h1 = MX(h), h2 = MX(h - h1), y = down (h1 + h2).  The output therefore
 * differs from the bf16 path's by the quantisation of x (about 5e-2 relative
 * L2 at the DS-like shape); it matches the exact layer evaluated on the same
 * quantised operands.  ws: moe355_workspace_bytes(d, T, MOE355_MODE_PREFILL_MX)
 * bytes, the error word at MOE355_PREFILL_ERR_BYTE (cleared by each call).
 * Limits: wfmt MOE355_W_MXFP4 (else MOE355_ENOTSUP), H a multiple of 256,
 * I a multiple of 128, both at most 16384, E <= 1024, T*H and T*k*I < 2^32.
 */
moe355_status moe355_expert_ffn_prefill_mx(const moe355_layer_desc* d, const void* x_bf16,
                                           int32_t T, const int32_t* topk_ids, const float* topk_w,
                                           const uint8_t* layer_w, const int32_t* perm,
                                           const int32_t* offsets, float* out, void* ws,
                                           size_t ws_bytes, hipStream_t stream);

/*
 * Prefill of n_layers consecutive MoE layers with the experts streamed from a
 * pinned host pool through whole-layer buffers [FT-zh, Core method and Method
 * steps: two whole-layer buffers; while the GPU computes layer l from one, a
 * transfer stream loads layer l+1 into the other over PCIe, then they swap;
 * FT-en, System Architecture: the buffer A / buffer B ping-pong].
 * For each layer l: copy host_pool's layer l (E * S bytes, device layout) into
 * a buffer by DMA on copy_stream, then on `stream` route T tokens from
 * logits[l], permute, and run moe355_expert_ffn_prefill on x[l] from that
 * buffer into out[l].  double_buffer != 0: layers alternate between buf0 and
 * buf1, so the copy of layer l+1 overlaps the compute of layer l; 0: buf0
 * alone, every copy waits for the previous layer's compute (buf1 unused).
 * host_pool: pinned host memory (hipHostMalloc) [n_layers * E * S]; buf0, buf1:
 * device [E * S]; logits, x, out: host arrays of n_layers device pointers
 * (fp32 [T, E], bf16 [T, H], fp32 [T, H]); topk_ids / topk_w / perm / offsets:
 * device scratch as for moe355_route and moe355_permute, reused by every layer;
 * ws / perm_ws: the MOE355_MODE_PREFILL and MOE355_MODE_PERMUTE workspaces.
 * When the call returns, `stream` holds the last layer's work and copy_stream
 * its copies.  Errors: MOE355_EINVAL for null pointers, a host_pool that is not
 * pinned host memory, or stream == copy_stream; MOE355_ECAPACITY for short
 * workspaces; otherwise as the calls above.
 */
moe355_status moe355_prefill_layers(const moe355_layer_desc* d, int32_t n_layers, int32_t T,
                                    const uint8_t* host_pool, uint8_t* buf0, uint8_t* buf1,
                                    const float* const* logits, const void* const* x,
                                    float* const* out, int32_t* topk_ids, float* topk_w,
                                    int32_t* perm, int32_t* offsets, void* ws, size_t ws_bytes,
                                    void* perm_ws, size_t perm_ws_bytes, int32_t double_buffer,
                                    hipStream_t stream, hipStream_t copy_stream);

/*
 * Unfused combine [FT-zh, Core method: the partial sums of a token's experts
 * merge into its output exactly; Edge0, section 2 "MoE routing": the output is
 * the routing-weighted sum over the selected experts]:
 * out[t, n] = sum_j topk_w[t, j] * y[t*k + j, n], j ascending, fp32 fused
 * multiply-adds.  The expert FFN calls fuse this step; this call serves callers
 * that hold per-pair outputs.  y: device fp32 [T*k, H]; topk_w: device fp32
 * [T, k]; out: device fp32 [T, H].  T = 0 enqueues nothing (the pointers may
 * then be null).  Errors: MOE355_EINVAL for null pointers, T < 0, H < 1 or k < 1.
 */
moe355_status moe355_combine(int32_t T, int32_t H, int32_t k, const float* y,
                             const float* topk_w, float* out, hipStream_t stream);

#define MOE355_MODE_DECODE   0
#define MOE355_MODE_PREFILL  1
#define MOE355_MODE_PERMUTE  2
#define MOE355_MODE_PREFILL_MX 3
/* Scratch bytes a call of the given mode needs for T tokens.  No page defines
 * this call; it sizes the caller-owned workspaces above.  Returns 0 for an
 * invalid descriptor, T < 0 or an unknown mode. */
size_t moe355_workspace_bytes(const moe355_layer_desc* d, int32_t T, int32_t mode);

#ifdef __cplusplus
}
#endif
#endif /* MOE355_H */
