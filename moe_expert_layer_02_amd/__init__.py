"""Python binding of libmoe355 (one MoE layer's forward pass on MI355X).

Argument marshalling only: every step runs in the HIP kernels of
``libmoe355.so``.  PyTorch supplies device memory and the stream.  Importing
this package fails loudly when the built library is missing; there is no CPU
path.  Build with ``python -m moe_expert_layer_02_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

from . import abi
from .abi import (LayerDesc, Cache, EvictPolicy, ClassifyOut, ROUTE_SOFTMAX_TOPK,
                  ROUTE_SIGMOID_GROUP, W_INT4_G64, W_MXFP4, MODE_DECODE, MODE_PREFILL,
                  MODE_PERMUTE, MODE_PREFILL_MX, Moe355Error, lib_path, load)
from .ops import (router_logits, route, dedup, classify_evict, cache_fill, cache_rebuild,
                  permute, expert_ffn_decode, decode_layer, decode_layer_static, route_plan,
                  evict_fill,
                  expert_ffn_prefill, expert_ffn_prefill_mx, quantize_mx, prefill_layers, combine,
                  workspace_bytes, pack_experts,
                  expert_bytes, version, check_build, error_word, check_error, ERR_WAIT,
                  ERR_F16_RANGE, DeviceCache, DeviceClassifyOut)

__all__ = [
    "LayerDesc", "Cache", "EvictPolicy", "ClassifyOut", "ROUTE_SOFTMAX_TOPK",
    "ROUTE_SIGMOID_GROUP", "W_INT4_G64", "W_MXFP4", "MODE_DECODE", "MODE_PREFILL", "MODE_PERMUTE",
    "MODE_PREFILL_MX", "expert_ffn_prefill_mx", "quantize_mx", "prefill_layers",
    "Moe355Error", "lib_path", "load", "router_logits", "route", "dedup", "classify_evict",
    "cache_fill", "cache_rebuild", "permute", "expert_ffn_decode", "decode_layer",
    "decode_layer_static", "route_plan",
    "evict_fill",
    "expert_ffn_prefill",
    "combine", "workspace_bytes", "pack_experts", "expert_bytes", "version", "check_build",
    "error_word", "check_error", "ERR_WAIT", "ERR_F16_RANGE", "DeviceCache", "DeviceClassifyOut",
]
