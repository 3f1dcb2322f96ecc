"""Shapes and parameters of the five synthetic MoE-layer workloads.

This module only names sizes and knobs; it performs none of the layer's
arithmetic.  The shapes follow the two model families the source pages
discuss: a Qwen-35B-A3B-like layer (Edge0 page, section 3.1 "Problem":
40 layers of 256 experts, int4 affine group-64, 1.77 MB per expert) and a
DeepSeek-style sigmoid-group layer (Edge0 page, section 2 "MoE routing";
FreeToken digest, "Background": 6 of 256 experts per token) with MXFP4
weights.
"""
from __future__ import annotations

from dataclasses import dataclass, field

ROUTE_SOFTMAX_TOPK = 0
ROUTE_SIGMOID_GROUP = 1

WFMT_INT4_G64 = 0
WFMT_MXFP4 = 1


@dataclass(frozen=True)
class Workload:
    cid: int                 # workload number, 1..5; seeds are 1000*cid + stream
    name: str
    hidden: int              # H
    inter: int               # I
    n_experts: int           # E
    top_k: int               # k
    route: int               # ROUTE_*
    n_group: int = 1
    topk_group: int = 1
    route_scale: float = 1.0
    wfmt: int = WFMT_INT4_G64
    n_layers: int = 1
    n_slots: int = 0         # HBM expert-cache slots (0: whole layer resident, no cache)
    t_decode: int = 0        # tokens per decode layer call
    t_prefill: int = 0       # tokens of the prefill layer call
    steps: int = 0           # decode steps in the routing trace
    zipf_alpha: float = 0.0
    keep_prob: float = 0.0
    q_num: int = 1           # miss split q = round(m * q_num / q_den), clamped to m
    q_den: int = 1
    shrink_step: int = -1    # step at whose start the slot budget changes
    shrink_slots: int = 0
    router_from_x: bool = False   # logits computed as x . W_r^T (tiny workload only)
    extra: dict = field(default_factory=dict)

    @property
    def victims_k(self) -> int:
        """Fixed capacity of the per-call victim / miss lists: min(T*k, E, N)."""
        t = max(self.t_decode, 1)
        n = self.n_slots if self.n_slots > 0 else self.n_experts
        return min(t * self.top_k, self.n_experts, n)


TINY = Workload(
    cid=1, name="tiny_int4_softmax_top2", hidden=256, inter=128, n_experts=16, top_k=2,
    route=ROUTE_SOFTMAX_TOPK, wfmt=WFMT_INT4_G64, n_layers=1, t_decode=4, t_prefill=4,
    router_from_x=True)

QWEN_DECODE = Workload(
    cid=2, name="qwen35b_like_decode_int4", hidden=2048, inter=512, n_experts=256, top_k=8,
    route=ROUTE_SOFTMAX_TOPK, wfmt=WFMT_INT4_G64, n_layers=40, n_slots=2048, t_decode=1,
    steps=256, zipf_alpha=1.1, keep_prob=0.8)

QWEN_PREFILL = Workload(
    cid=3, name="qwen35b_like_prefill_int4", hidden=2048, inter=512, n_experts=256, top_k=8,
    route=ROUTE_SOFTMAX_TOPK, wfmt=WFMT_INT4_G64, n_layers=1, t_prefill=8192)

DS_DECODE = Workload(
    cid=4, name="dsv_like_decode_mxfp4", hidden=4096, inter=2048, n_experts=256, top_k=6,
    route=ROUTE_SIGMOID_GROUP, n_group=8, topk_group=4, route_scale=2.5, wfmt=WFMT_MXFP4,
    n_layers=24, n_slots=1024, t_decode=16, steps=128, zipf_alpha=1.0, keep_prob=0.6)

DS_STRESS = Workload(
    cid=5, name="dsv_like_prefill_and_cache_stress_mxfp4", hidden=4096, inter=2048,
    n_experts=256, top_k=6, route=ROUTE_SIGMOID_GROUP, n_group=8, topk_group=4,
    route_scale=2.5, wfmt=WFMT_MXFP4, n_layers=24, n_slots=1024, t_decode=16,
    t_prefill=16384, steps=512, zipf_alpha=1.0, keep_prob=0.6, q_num=527, q_den=773,
    shrink_step=256, shrink_slots=384)

ALL = {w.cid: w for w in (TINY, QWEN_DECODE, QWEN_PREFILL, DS_DECODE, DS_STRESS)}

# Single-stream (one token per step) DeepSeek-style decode trace, for the miss
# rate versus cache size replay: the pages replay the routing of single agent
# sessions, and a 16-token batch's working set (about 56 experts per layer call)
# exceeds small caches by itself.
DS_DECODE_SINGLE = Workload(
    cid=10, name="dsv_like_decode_single_stream", hidden=4096, inter=2048, n_experts=256,
    top_k=6, route=ROUTE_SIGMOID_GROUP, n_group=8, topk_group=4, route_scale=2.5,
    wfmt=WFMT_MXFP4, n_layers=24, n_slots=1024, t_decode=1, steps=256, zipf_alpha=1.0,
    keep_prob=0.6)


def seed(cid: int, stream: int) -> int:
    """Seed of one input stream: 0 weights, 1 activations, 2 logits / trace."""
    return 1000 * cid + stream
