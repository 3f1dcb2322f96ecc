"""Decode-time expert miss rate versus cache size, replayed on routing traces.

[FT-zh, Results: the decode expert-cache miss rate under same-capacity routing
replay, the cache being 37 % / 11 % of the expert pool, for the global LRU
against static hot-expert pinning and static whole-layer placement; FT-en,
Performance Evaluation, Figure 4b: miss rate versus cache size as a
percentage of the pool, three placement policies on identical traces.]

* ``lru_misses`` replays a trace through the library's own bookkeeping call
  (``moe355_route`` + ``moe355_classify_evict`` with pure fill, q = m) on the
  GPU and returns each call's distinct-expert and miss counts from the
  device's count arrays.
* ``hot_pinned_misses`` and ``layer_static_misses`` are the two static
  placements the pages compare against, evaluated on the host: a fixed set of
  the N most frequently routed (layer, expert) pairs of the trace (ties to the
  lower layer, then expert), or whole layers 0, 1, ... as long as they fit in
  N slots.  Neither changes during decode, so their misses are a set
  membership count.

A trace is router logits [steps, L, T, E]; a call's distinct experts are the
distinct ids its T tokens route to.  The miss rate is the sum of misses over
the sum of distinct experts.
"""
from __future__ import annotations

import numpy as np


def lru_misses(desc, logits, n_slots: int, K: int, steps=None):
    """Global LRU over every layer: per-call (distinct, misses) [steps, L, 2] int64,
    and the routed ids [steps, L, T, k] the GPU router produced."""
    import torch
    from . import ops
    from .abi import EvictPolicy
    S, L, T, E = logits.shape
    steps = S if steps is None else steps
    cache = ops.DeviceCache(n_slots, L, E, 1, with_data=False)
    policy = EvictPolicy(K, 1, 1)
    cap = max(K, min(T * desc.top_k, E))
    out = ops.DeviceClassifyOut(cap, pair_capacity=T * desc.top_k)
    lg = torch.from_numpy(np.ascontiguousarray(logits[:steps])).cuda()
    wt = torch.empty((T, desc.top_k), dtype=torch.float32, device="cuda")
    counts = torch.empty((steps, L, 6), dtype=torch.int32, device="cuda")
    routed = torch.empty((steps, L, T, desc.top_k), dtype=torch.int32, device="cuda")
    for s in range(steps):
        for l in range(L):
            ops.route(desc, lg[s, l], routed[s, l], wt)
            ops.classify_evict(cache, l, s * L + l + 1, routed[s, l], policy, out)
            counts[s, l].copy_(out.counts)
    c = counts.cpu().numpy().astype(np.int64)
    return np.stack([c[..., 0], c[..., 2]], axis=-1), routed.cpu().numpy()


def distinct_sets(routed_ids):
    """Per call, the sorted distinct (layer-local) expert ids: routed_ids [steps, L, T, k]."""
    S, L = routed_ids.shape[:2]
    return [[np.unique(routed_ids[s, l]) for l in range(L)] for s in range(S)]


def hot_pinned_misses(routed_ids, n_experts: int, n_slots: int):
    """Static hot-expert pinning: per-call (distinct, misses) [steps, L, 2]."""
    sets = distinct_sets(routed_ids)
    S, L = len(sets), len(sets[0])
    freq = np.zeros(L * n_experts, dtype=np.int64)
    for s in range(S):
        for l in range(L):
            freq[l * n_experts + sets[s][l]] += 1
    # the n_slots most frequent (layer, expert) pairs; ties to the lower global id
    order = np.lexsort((np.arange(freq.size), -freq))
    pinned = np.zeros(freq.size, dtype=bool)
    pinned[order[:min(n_slots, freq.size)]] = True
    out = np.zeros((S, L, 2), dtype=np.int64)
    for s in range(S):
        for l in range(L):
            u = sets[s][l]
            out[s, l] = (u.size, int((~pinned[l * n_experts + u]).sum()))
    return out


def layer_static_misses(routed_ids, n_experts: int, n_slots: int):
    """Static whole-layer placement: layers 0 .. n_slots // E - 1 resident."""
    sets = distinct_sets(routed_ids)
    S, L = len(sets), len(sets[0])
    resident = min(L, n_slots // n_experts)
    out = np.zeros((S, L, 2), dtype=np.int64)
    for s in range(S):
        for l in range(L):
            u = sets[s][l].size
            out[s, l] = (u, 0 if l < resident else u)
    return out


def miss_rate(per_call) -> float:
    per_call = np.asarray(per_call)
    return float(per_call[..., 1].sum() / max(per_call[..., 0].sum(), 1))
