"""The miss-rate replay's global LRU runs through the library's routing and
bookkeeping calls on the GPU: every call's distinct and miss counts, and the
routed ids, equal the oracle's routing and cache simulator, at several cache
sizes (fractions of the expert pool), on the Qwen-like trace and the
single-stream DS-like trace."""
import numpy as np
import pytest

from oracle import cache as ocache
from oracle import route as oroute
from workloads import configs as C
from workloads import traces as tr

from gpu_common import desc_of, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cid,frac", [(2, 0.05), (2, 0.37), (10, 0.11), (10, 0.5)])
def test_lru_replay_matches_simulator(cid, frac):
    from moe_expert_layer_02_amd import replay
    w = C.ALL[cid] if cid in C.ALL else C.DS_DECODE_SINGLE
    steps = 24
    trace = tr.DecodeTrace(w, steps)
    L, E = w.n_layers, w.n_experts
    N = int(frac * L * E)
    K = min(w.t_decode * w.top_k, E, N)
    got, routed = replay.lru_misses(desc_of(w), trace.logits, N, K)
    sim = ocache.CacheSim(N, L, E)
    for s in range(steps):
        for l in range(L):
            ids, _ = oroute.route(trace.logits[s, l], w.top_k, w.route, w.n_group, w.topk_group,
                                  w.route_scale)
            assert np.array_equal(routed[s, l], ids), (s, l)
            c = sim.classify_evict(l, s * L + l + 1, ids, K)["counts"]
            assert got[s, l].tolist() == [c[0], c[2]], (s, l)
    say(f"{w.name} at {frac:.0%} of the pool ({N} slots): LRU miss rate "
        f"{replay.miss_rate(got):.3f}, {steps * L} calls equal to the simulator")
