"""Pins of the oracle's cache integer path: the pages' worked examples, exact
rounding of the miss split, and agreement with an independent ordered-dict LRU
on random traces (including a mid-run shrink)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle.cache import CacheSim, q_split, slots_for_budget
from oracle.lru_reference import OrderedLRU

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def _ratio(b_p, b_h):
    f = Fraction(str(b_p)) / Fraction(str(b_h))
    return f.numerator, f.denominator


@pytest.mark.parametrize("case", GOLD["q_split"], ids=lambda c: f"m{c['m']}")
def test_q_split_worked_examples(case):
    num, den = _ratio(case["b_p"], case["b_h"])
    assert q_split(case["m"], num, den) == case["q"]


def test_q_split_is_round_half_up_and_clamped():
    for num, den in [(527, 773), (1, 2), (1, 1), (118, 475), (3, 1), (0, 5)]:
        for m in range(0, 1200):
            exact = Fraction(m * num, den)
            want = min(m, int(exact + Fraction(1, 2)))   # floor(x + 1/2)
            assert q_split(m, num, den) == want, (num, den, m)
    # pure fill when the two bandwidths are equal
    assert all(q_split(m, 1, 1) == m for m in range(200))
    # the closed form for 52.7/77.3 used by the cache-pressure workload
    for m in range(0, 773):
        assert q_split(m, 527, 773) == (1054 * m + 773) // 1546


@pytest.mark.parametrize("case", GOLD["slot_budget"], ids=lambda c: str(c["budget_gb"]))
def test_slot_budget_examples(case):
    scale = 1000
    assert slots_for_budget(int(case["budget_gb"] * scale), int(case["slot_gb"] * scale)) == case["slots"]


def test_single_pass_lru_example():
    ex = GOLD["lru_single_pass"]
    E = 16
    sim = CacheSim(n_slots=4, n_layers=1, n_experts=E)
    for slot, (e, ts) in enumerate(zip([4, 5, 6, 7], ex["slot_ts"])):
        sim.table[e] = slot
        sim.owner[slot] = e
        sim.ts[slot] = ts
    tick = 31
    out = sim.classify_evict(0, tick, [9, 10], K=ex["q"], q_num=1, q_den=1)
    victim_ts = [ex["slot_ts"][v] for v in out["victims"]]
    assert victim_ts == ex["victim_ts"]
    assert out["fill_slot"] == out["victims"] and out["fill_expert"] == [9, 10]
    assert [int(sim.ts[v]) for v in out["victims"]] == [tick, tick]
    assert sorted(int(sim.ts[s]) for s in range(4) if s not in out["victims"]) == ex["untouched_ts"]
    assert sim.table[4] == -1 and sim.table[5] == -1 and sim.table[9] >= 0 and sim.table[10] >= 0


def test_hits_are_touched_and_never_victims():
    sim = CacheSim(n_slots=3, n_layers=1, n_experts=8)
    sim.classify_evict(0, 1, [0, 1, 2], K=3)
    out = sim.classify_evict(0, 2, [0, 3], K=3)
    assert out["hit_expert"] == [0] and out["miss"] == [3]
    assert sim.table[0] == out["hit_slot"][0]
    assert out["hit_slot"][0] not in out["victims"]
    assert sim.ts[out["hit_slot"][0]] == 2


def test_in_place_set_when_victims_run_out():
    # every slot is a hit of this call, so no victim is eligible: misses go in place
    sim = CacheSim(n_slots=2, n_layers=1, n_experts=8)
    sim.classify_evict(0, 1, [0, 1], K=2)
    out = sim.classify_evict(0, 2, [0, 1, 5, 6], K=4)
    assert out["victims"] == [] and out["fill_expert"] == [] and out["inplace"] == [5, 6]
    assert out["counts"] == [4, 2, 2, 0, 2, 0]


def _random_trace(rng, L, E, T, k, steps, hot):
    for step in range(steps):
        for l in range(L):
            p = np.arange(1, E + 1, dtype=float) ** -1.1
            p = p[rng.permutation(E)] if hot is None else p
            p /= p.sum()
            ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)])
            yield step, l, ids


@pytest.mark.parametrize("N,L,E,T,k,num,den", [
    (24, 4, 16, 1, 4, 1, 1),
    (10, 3, 32, 4, 3, 1, 2),
    (40, 5, 64, 2, 6, 527, 773),
    (7, 2, 16, 3, 2, 3, 1),
])
def test_sim_matches_ordered_dict_lru(N, L, E, T, k, num, den):
    rng = np.random.default_rng(N * 131 + E)
    sim = CacheSim(N, L, E)
    ref = OrderedLRU(N, E)
    K = min(T * k, E, N)
    for step, l, ids in _random_trace(rng, L, E, T, k, 30, hot=None):
        tick = step * L + l + 1
        out = sim.classify_evict(l, tick, ids, K, num, den)
        q = q_split(out["counts"][2], num, den)
        r = ref.call(l, ids.ravel(), K, q)
        for key in ("hit_expert", "fill_expert", "fill_slot", "inplace", "victims"):
            assert out[key] == r[key], (step, l, key)
    table = {int(g): int(s) for g, s in enumerate(sim.table) if s >= 0}
    assert table == ref.table()


def test_sim_rebuild_matches_ordered_dict_shrink():
    N, L, E, T, k = 30, 3, 32, 2, 4
    rng = np.random.default_rng(5)
    sim, ref = CacheSim(N, L, E), OrderedLRU(N, E)
    K = min(T * k, E, N)
    trace = list(_random_trace(rng, L, E, T, k, 40, hot=None))
    for i, (step, l, ids) in enumerate(trace):
        if i == len(trace) // 2:
            sim, ref = sim.rebuild(12), ref.shrink(12)
            K = min(T * k, E, 12)
            assert {int(g): int(s) for g, s in enumerate(sim.table) if s >= 0} == ref.table()
        tick = step * L + l + 1
        out = sim.classify_evict(l, tick, ids, K)
        r = ref.call(l, ids.ravel(), K, out["counts"][2])
        for key in ("hit_expert", "fill_expert", "fill_slot", "inplace", "victims"):
            assert out[key] == r[key]


def test_rebuild_keeps_most_recent_and_packs_in_slot_order():
    sim = CacheSim(6, 1, 16)
    ts = [5, 0, 9, 7, 9, 3]
    owners = [0, -1, 2, 3, 4, 5]
    for s in range(6):
        sim.ts[s], sim.owner[s] = ts[s], owners[s]
        if owners[s] >= 0:
            sim.table[owners[s]] = s
    new = sim.rebuild(3)
    # occupied by (ts, slot): (3,5) (5,0) (7,3) (9,2) (9,4) -> keep the last three: slots 2, 3, 4
    assert new.owner.tolist() == [2, 3, 4]
    assert new.ts.tolist() == [9, 7, 9]
    assert new.table[2] == 0 and new.table[3] == 1 and new.table[4] == 2 and new.table[0] == -1
    grow = sim.rebuild(8)
    assert grow.owner.tolist() == [0, 2, 3, 4, 5, -1, -1, -1]


def test_moves_of_rebuild_hand_example():
    """Occupied (ts, slot): (3,5) (5,0) (7,3) (9,2) (9,4); keeping three moves the
    bytes of old slots 2, 3, 4 to new slots 0, 1, 2; keeping all moves every
    occupied slot down to its rank in slot order."""
    sim = CacheSim(6, 1, 16)
    for s, (t, o) in enumerate(zip([5, 0, 9, 7, 9, 3], [0, -1, 2, 3, 4, 5])):
        sim.ts[s], sim.owner[s] = t, o
        if o >= 0:
            sim.table[o] = s
    assert sim.moves_of_rebuild(3) == [(2, 0), (3, 1), (4, 2)]
    assert sim.moves_of_rebuild(8) == [(0, 0), (2, 1), (3, 2), (4, 3), (5, 4)]
    assert sim.moves_of_rebuild(1) == [(4, 0)]      # ts tie (9, 2) < (9, 4): slot 4 is newest


@pytest.mark.parametrize("n_new", [1, 7, 12, 30, 45])
def test_moves_of_rebuild_match_ordered_dict_shrink(n_new):
    """The bytes a rebuild moves are the renumbering the textbook LRU's shrink
    applies to its kept entries, on a cache shaped by a random trace."""
    N, L, E, T, k = 30, 3, 32, 2, 4
    rng = np.random.default_rng(n_new)
    sim, ref = CacheSim(N, L, E), OrderedLRU(N, E)
    K = min(T * k, E, N)
    for step, l, ids in _random_trace(rng, L, E, T, k, 12, hot=None):
        out = sim.classify_evict(l, step * L + l + 1, ids, K)
        ref.call(l, ids.ravel(), K, out["counts"][2])
    moves = sim.moves_of_rebuild(n_new)
    assert moves == ref.shrink(n_new).moved
    # every move carries an occupied slot to a distinct new slot, in slot order
    assert [n for _, n in moves] == list(range(len(moves)))
    assert all(sim.owner[o] >= 0 for o, _ in moves)
