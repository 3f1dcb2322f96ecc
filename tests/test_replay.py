"""The miss-rate replay's static placements on hand-built traces (host only):
hot-expert pinning keeps the most frequently routed (layer, expert) pairs,
ties to the lower id; whole-layer placement keeps layers 0, 1, ... while they
fit."""
import numpy as np

from moe_expert_layer_02_amd import replay


def _trace():
    # 3 steps, 2 layers, 1 token, k = 2, E = 4
    return np.array([[[[0, 1]], [[2, 3]]],
                     [[[0, 2]], [[2, 1]]],
                     [[[1, 0]], [[3, 2]]]], dtype=np.int32)


def test_hot_pinned_hand_example():
    ids = _trace()
    # frequencies: layer 0: e0 3, e1 2, e2 1; layer 1: e2 3, e3 2, e1 1
    # 2 slots pin (0, 0) and (1, 2); 3 slots add (0, 1) (global id 1 < 7)
    r2 = replay.hot_pinned_misses(ids, 4, 2)
    assert r2[..., 0].tolist() == [[2, 2], [2, 2], [2, 2]]
    assert r2[..., 1].tolist() == [[1, 1], [1, 1], [1, 1]]
    r3 = replay.hot_pinned_misses(ids, 4, 3)
    assert r3[..., 1].tolist() == [[0, 1], [1, 1], [0, 1]]
    assert replay.miss_rate(r3) == 4 / 12
    assert replay.miss_rate(replay.hot_pinned_misses(ids, 4, 8)) == 0.0
    assert replay.miss_rate(replay.hot_pinned_misses(ids, 4, 0)) == 1.0


def test_layer_static_hand_example():
    ids = _trace()
    assert replay.miss_rate(replay.layer_static_misses(ids, 4, 3)) == 1.0     # no whole layer fits
    r = replay.layer_static_misses(ids, 4, 4)                                 # layer 0 resident
    assert r[..., 1].tolist() == [[0, 2], [0, 2], [0, 2]]
    assert replay.miss_rate(replay.layer_static_misses(ids, 4, 8)) == 0.0


def test_duplicate_ids_of_a_call_count_once():
    ids = np.array([[[[1, 2], [2, 3]]]], dtype=np.int32)       # 1 step, 1 layer, 2 tokens
    r = replay.layer_static_misses(ids, 4, 0)
    assert r.tolist() == [[[3, 3]]]
