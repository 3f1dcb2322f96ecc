"""Torch-tensor front end of the libmoe355 calls.

Each function takes device tensors, hands their addresses and the current HIP
stream to the C call of the same name, and raises ``Moe355Error`` on a
non-zero status.  Nothing here computes any part of the layer.
"""
from __future__ import annotations

import ctypes

import torch

from .abi import (Cache, ClassifyOut, EvictPolicy, LayerDesc, MODE_DECODE, MODE_PERMUTE,
                  MODE_PREFILL, MODE_PREFILL_MX, Moe355Error, check, load)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmoe355 takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libmoe355 takes contiguous tensors")
    return t.data_ptr()


def _pool_ptr(t) -> int:
    """The expert pool: device memory, or pinned host memory (the host tier, read
    by the kernels over PCIe)."""
    if t.is_cuda:
        return _ptr(t)
    if not t.is_pinned():
        raise ValueError("libmoe355: a host expert pool must be pinned memory")
    if not t.is_contiguous():
        raise ValueError("libmoe355 takes contiguous tensors")
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def version() -> str:
    return load().moe355_version().decode()


def check_build() -> str:
    """The loaded library's source hash must be the tree's: raises otherwise."""
    from .build import source_hash
    v = version()
    want = source_hash()
    if not v.endswith("src:" + want):
        raise Moe355Error(-1, "check_build",
                          f"the loaded library ({v}) was not built from these sources (src:{want}); "
                          "rebuild with python -m moe_expert_layer_02_amd.build")
    return v


DECODE_ERR_BYTE = 4608     # MOE355_DECODE_ERR_BYTE
PREFILL_ERR_BYTE = 0       # MOE355_PREFILL_ERR_BYTE
ERR_WAIT = 1
ERR_F16_RANGE = 2


def error_word(ws, mode: int = MODE_DECODE) -> int:
    """The error word of a decode or prefill workspace (synchronises)."""
    at = DECODE_ERR_BYTE if mode == MODE_DECODE else PREFILL_ERR_BYTE   # both prefill forms
    return int(ws[at:at + 4].view(torch.int32).item()) & 0xFFFFFFFF


def check_error(ws, mode: int = MODE_DECODE, what: str = "") -> None:
    """Raise if the workspace's error word records an invalid call (synchronises)."""
    e = error_word(ws, mode)
    if e:
        why = []
        if e & ERR_WAIT:
            why.append("a bounded in-kernel wait gave up")
        if e & ERR_F16_RANGE:
            why.append("an int4-path activation or intermediate left f16's range")
        raise Moe355Error(-2, what or "check_error", f"error word {e:#x}: " + "; ".join(why))


def expert_bytes(desc: LayerDesc) -> int:
    return int(load().moe355_expert_bytes(ctypes.byref(desc)))


def pack_experts(desc: LayerDesc, src, dst, n: int, stream=None):
    """n expert blobs from the canonical layout (src) to the device layout (dst)."""
    _need(src, torch.uint8, "src")
    _need(dst, torch.uint8, "dst")
    S = expert_bytes(desc)
    if src.numel() < n * S or dst.numel() < n * S:
        raise ValueError(f"pack_experts: buffers hold fewer than {n} experts of {S} bytes")
    check(load().moe355_pack_experts(ctypes.byref(desc), _ptr(src), _ptr(dst), n, _stream(stream)),
          "moe355_pack_experts")


def workspace_bytes(desc: LayerDesc, T: int, mode: int) -> int:
    return int(load().moe355_workspace_bytes(ctypes.byref(desc), T, mode))


def router_logits(desc, x_bf16, w_router, logits, stream=None):
    _need(x_bf16, torch.bfloat16, "x")
    _need(w_router, torch.float32, "w_router")
    _need(logits, torch.float32, "logits")
    T = x_bf16.shape[0]
    check(load().moe355_router_logits(ctypes.byref(desc), _ptr(x_bf16), _ptr(w_router), T,
                                      _ptr(logits), _stream(stream)), "moe355_router_logits")


def route(desc, logits, topk_ids, topk_w, stream=None):
    _need(logits, torch.float32, "logits")
    _need(topk_ids, torch.int32, "topk_ids")
    _need(topk_w, torch.float32, "topk_w")
    T = logits.shape[0]
    check(load().moe355_route(ctypes.byref(desc), _ptr(logits), T, _ptr(topk_ids), _ptr(topk_w),
                              _stream(stream)), "moe355_route")


class DeviceClassifyOut:
    """Caller-owned per-call lists (``capacity`` int32 each) plus counts[6]."""

    NAMES = ("uniq", "hit_expert", "hit_slot", "miss", "fill_expert", "fill_slot", "inplace",
             "victims")

    def __init__(self, capacity: int, pair_capacity: int = 1024, device="cuda"):
        self.capacity = capacity
        self.buf = torch.full((len(self.NAMES), max(capacity, 1)), -1, dtype=torch.int32,
                              device=device)
        self.counts = torch.zeros(6, dtype=torch.int32, device=device)
        self.plan = torch.zeros((max(capacity, 1), 4), dtype=torch.int32, device=device)
        self.pairs = torch.zeros(max(pair_capacity, 1), dtype=torch.int32, device=device)
        self.struct = ClassifyOut(*[self.buf[i].data_ptr() for i in range(len(self.NAMES))],
                                  self.counts.data_ptr(), capacity, self.plan.data_ptr(),
                                  self.pairs.data_ptr(), pair_capacity)

    def list(self, name: str):
        return self.buf[self.NAMES.index(name)]

    def host(self) -> dict:
        """Copy the lists to the host, trimmed to their counts (synchronises)."""
        b = self.buf.cpu()
        c = self.counts.cpu().tolist()
        n = {"uniq": c[0], "hit_expert": c[1], "hit_slot": c[1], "miss": c[2],
             "fill_expert": c[3], "fill_slot": c[3], "inplace": c[4], "victims": c[5]}
        out = {k: b[i, :n[k]].tolist() for i, k in enumerate(self.NAMES)}
        out["counts"] = c
        out["plan"] = self.plan[:c[0]].cpu().tolist()
        out["pairs"] = self.pairs.cpu().tolist()
        return out


class DeviceCache:
    """The HBM expert cache: slot table, owner, timestamps and slot bytes."""

    def __init__(self, n_slots: int, n_layers: int, n_experts: int, slot_bytes: int,
                 device="cuda", with_data: bool = True):
        self.table = torch.full((n_layers * n_experts,), -1, dtype=torch.int32, device=device)
        self.owner = torch.full((n_slots,), -1, dtype=torch.int32, device=device)
        self.ts = torch.zeros((n_slots,), dtype=torch.int64, device=device)
        self.data = (torch.empty((n_slots * slot_bytes,), dtype=torch.uint8, device=device)
                     if with_data else None)
        self.struct = Cache(n_slots, n_layers, n_experts, slot_bytes, self.table.data_ptr(),
                            self.owner.data_ptr(), self.ts.data_ptr(),
                            self.data.data_ptr() if self.data is not None else None)

    @property
    def n_slots(self) -> int:
        return self.struct.n_slots


def dedup(ids, n_experts: int, out: DeviceClassifyOut, stream=None):
    _need(ids, torch.int32, "ids")
    check(load().moe355_dedup(_ptr(ids), ids.numel(), n_experts, ctypes.byref(out.struct),
                              _stream(stream)), "moe355_dedup")


def classify_evict(cache: DeviceCache, layer: int, tick: int, ids, policy: EvictPolicy,
                   out: DeviceClassifyOut, stream=None):
    _need(ids, torch.int32, "ids")
    check(load().moe355_classify_evict(ctypes.byref(cache.struct), layer, tick, _ptr(ids),
                                       ids.numel(), ctypes.byref(policy),
                                       ctypes.byref(out.struct), _stream(stream)),
          "moe355_classify_evict")


def cache_fill(cache: DeviceCache, pool, layer: int, out: DeviceClassifyOut, max_fill: int,
               stream=None):
    _need(pool, torch.uint8, "pool")
    check(load().moe355_cache_fill(ctypes.byref(cache.struct), _pool_ptr(pool), layer,
                                   ctypes.byref(out.struct), max_fill, _stream(stream)),
          "moe355_cache_fill")


def cache_rebuild(src: DeviceCache, dst: DeviceCache, stream=None):
    check(load().moe355_cache_rebuild(ctypes.byref(src.struct), ctypes.byref(dst.struct),
                                      _stream(stream)), "moe355_cache_rebuild")


def permute(desc, topk_ids, perm, offsets, ws, stream=None):
    _need(topk_ids, torch.int32, "topk_ids")
    T = topk_ids.shape[0]
    check(load().moe355_permute(ctypes.byref(desc), _ptr(topk_ids), T, _ptr(perm), _ptr(offsets),
                                _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
          "moe355_permute")


def expert_ffn_decode(desc, x_bf16, topk_ids, topk_w, cache, pool, layer: int,
                      experts: DeviceClassifyOut, out, ws, stream=None):
    _need(x_bf16, torch.bfloat16, "x")
    _need(out, torch.float32, "out")
    T = x_bf16.shape[0]
    cptr = ctypes.byref(cache.struct) if cache is not None else None
    check(load().moe355_expert_ffn_decode(ctypes.byref(desc), _ptr(x_bf16), T, _ptr(topk_ids),
                                          _ptr(topk_w), cptr, _pool_ptr(pool), layer,
                                          ctypes.byref(experts.struct), _ptr(out), _ptr(ws),
                                          ws.numel() * ws.element_size(), _stream(stream)),
          "moe355_expert_ffn_decode")


def decode_layer(desc, cache: DeviceCache, pool, layer: int, tick_base, tick_add: int, logits,
                 x_bf16, policy: EvictPolicy, topk_ids, topk_w, lists: DeviceClassifyOut, out, ws,
                 stream=None):
    """route + classify_evict + expert FFN (fill-through) for one layer call."""
    _need(logits, torch.float32, "logits")
    _need(x_bf16, torch.bfloat16, "x")
    if tick_base is not None:
        _need(tick_base, torch.int64, "tick_base")
    T = x_bf16.shape[0]
    check(load().moe355_decode_layer(ctypes.byref(desc), ctypes.byref(cache.struct), _pool_ptr(pool),
                                     layer, _ptr(tick_base), tick_add, _ptr(logits), _ptr(x_bf16),
                                     T, ctypes.byref(policy), _ptr(topk_ids), _ptr(topk_w),
                                     ctypes.byref(lists.struct), _ptr(out), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)),
          "moe355_decode_layer")


def decode_layer_static(desc, cache: DeviceCache, pool, layer: int, tick_base, tick_add: int,
                        logits, x_bf16, policy: EvictPolicy, topk_ids, topk_w,
                        lists: DeviceClassifyOut, out, err_word, stream=None):
    """decode_layer with the library's fixed per-GPU scratch instead of a workspace;
    err_word: a device int32 [1] the call ORs its error bits into."""
    _need(logits, torch.float32, "logits")
    _need(x_bf16, torch.bfloat16, "x")
    _need(err_word, torch.int32, "err_word")
    if tick_base is not None:
        _need(tick_base, torch.int64, "tick_base")
    T = x_bf16.shape[0]
    check(load().moe355_decode_layer_static(ctypes.byref(desc), ctypes.byref(cache.struct),
                                            _pool_ptr(pool), layer, _ptr(tick_base), tick_add,
                                            _ptr(logits), _ptr(x_bf16), T, ctypes.byref(policy),
                                            _ptr(topk_ids), _ptr(topk_w), ctypes.byref(lists.struct),
                                            _ptr(out), _ptr(err_word), _stream(stream)),
          "moe355_decode_layer_static")


def route_plan(desc, cache: DeviceCache, layer: int, logits, topk_ids, topk_w,
               lists: DeviceClassifyOut, stream=None):
    """Route + dedup + hit/miss + FFN plan (hits from slots, misses from the pool)."""
    _need(logits, torch.float32, "logits")
    T = logits.shape[0]
    check(load().moe355_route_plan(ctypes.byref(desc), ctypes.byref(cache.struct), layer,
                                   _ptr(logits), T, _ptr(topk_ids), _ptr(topk_w),
                                   ctypes.byref(lists.struct), _stream(stream)),
          "moe355_route_plan")


def evict_fill(desc, cache: DeviceCache, pool, layer: int, tick_base, tick_add: int, topk_ids,
               policy: EvictPolicy, lists: DeviceClassifyOut, stream=None):
    """Hit stamps, K LRU victims, slot update and the pool -> slot copy of a planned call."""
    _need(topk_ids, torch.int32, "topk_ids")
    if tick_base is not None:
        _need(tick_base, torch.int64, "tick_base")
    T = topk_ids.shape[0]
    check(load().moe355_evict_fill(ctypes.byref(desc), ctypes.byref(cache.struct), _pool_ptr(pool),
                                   layer, _ptr(tick_base), tick_add, _ptr(topk_ids), T,
                                   ctypes.byref(policy), ctypes.byref(lists.struct),
                                   _stream(stream)), "moe355_evict_fill")


def expert_ffn_prefill(desc, x_bf16, topk_ids, topk_w, layer_w, perm, offsets, out, ws,
                       stream=None):
    _need(x_bf16, torch.bfloat16, "x")
    _need(out, torch.float32, "out")
    T = x_bf16.shape[0]
    check(load().moe355_expert_ffn_prefill(ctypes.byref(desc), _ptr(x_bf16), T, _ptr(topk_ids),
                                           _ptr(topk_w), _ptr(layer_w), _ptr(perm), _ptr(offsets),
                                           _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                           _stream(stream)), "moe355_expert_ffn_prefill")


def quantize_mx(x_bf16, codes, scales, stream=None):
    """MX FP8 E4M3 codes [rows, cols] and scale bytes [rows, cols / 32] of bf16 x."""
    _need(x_bf16, torch.bfloat16, "x")
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.uint8, "scales")
    rows, cols = x_bf16.shape
    if codes.numel() < rows * cols or scales.numel() < rows * cols // 32:
        raise ValueError("quantize_mx: output buffers too small")
    check(load().moe355_quantize_mx(_ptr(x_bf16), rows, cols, _ptr(codes), _ptr(scales),
                                    _stream(stream)), "moe355_quantize_mx")


def expert_ffn_prefill_mx(desc, x_bf16, topk_ids, topk_w, layer_w, perm, offsets, out, ws,
                          stream=None):
    """Prefill expert FFN for MXFP4 experts on the fp4 x fp8 matrix cores."""
    _need(x_bf16, torch.bfloat16, "x")
    _need(out, torch.float32, "out")
    T = x_bf16.shape[0]
    check(load().moe355_expert_ffn_prefill_mx(ctypes.byref(desc), _ptr(x_bf16), T, _ptr(topk_ids),
                                              _ptr(topk_w), _ptr(layer_w), _ptr(perm),
                                              _ptr(offsets), _ptr(out), _ptr(ws),
                                              ws.numel() * ws.element_size(), _stream(stream)),
          "moe355_expert_ffn_prefill_mx")


def prefill_layers(desc, host_pool, bufs, logits, xs, outs, topk_ids, topk_w, perm, offsets, ws,
                   perm_ws, double_buffer: bool, stream=None, copy_stream=None):
    """Prefill of len(logits) layers, experts streamed from a pinned host pool
    through one or two whole-layer device buffers (copies on copy_stream)."""
    if host_pool.is_cuda or not host_pool.is_pinned():
        raise ValueError("prefill_layers: host_pool must be pinned host memory")
    n = len(logits)
    if not (len(xs) == len(outs) == n):
        raise ValueError("prefill_layers: one logits, x and out tensor per layer")
    for t in xs:
        _need(t, torch.bfloat16, "x")
    arr = ctypes.c_void_p * n
    lp, xp, op = arr(*[_ptr(t) for t in logits]), arr(*[_ptr(t) for t in xs]), arr(*[_ptr(t) for t in outs])
    T = xs[0].shape[0]
    if copy_stream is None:
        raise ValueError("prefill_layers: a copy stream is required")
    check(load().moe355_prefill_layers(ctypes.byref(desc), n, T, host_pool.data_ptr(), _ptr(bufs[0]),
                                       _ptr(bufs[1]) if double_buffer else None, lp, xp, op,
                                       _ptr(topk_ids), _ptr(topk_w), _ptr(perm), _ptr(offsets),
                                       _ptr(ws), ws.numel() * ws.element_size(), _ptr(perm_ws),
                                       perm_ws.numel() * perm_ws.element_size(),
                                       1 if double_buffer else 0, _stream(stream),
                                       ctypes.c_void_p(copy_stream.cuda_stream)),
          "moe355_prefill_layers")


def combine(y, topk_w, out, stream=None):
    T, k = topk_w.shape
    H = out.shape[1]
    check(load().moe355_combine(T, H, k, _ptr(y), _ptr(topk_w), _ptr(out), _stream(stream)),
          "moe355_combine")
