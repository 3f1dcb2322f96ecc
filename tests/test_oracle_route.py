"""Pins of the oracle's routers: brute force over every subset on tiny inputs,
library softmax / sigmoid for the special cases, and the weight sums."""
import itertools

import numpy as np
import pytest
from scipy.special import expit, softmax

from oracle import route


def _rand_logits(seed, T, E):
    return np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32)


@pytest.mark.parametrize("seed", range(5))
def test_softmax_topk_brute_force(seed):
    lg = _rand_logits(seed, 6, 16)
    ids, w = route.softmax_topk(lg, 2)
    for t in range(lg.shape[0]):
        best = max(itertools.combinations(range(16), 2),
                   key=lambda c: sum(float(lg[t, i]) for i in c))
        assert set(ids[t].tolist()) == set(best)
        assert lg[t, ids[t, 0]] >= lg[t, ids[t, 1]]
        # softmax over all E, then renormalise over the kept pair
        p = softmax(lg[t].astype(np.float64))
        ref = p[ids[t]] / p[ids[t]].sum()
        np.testing.assert_allclose(w[t], ref, rtol=1e-12)
        assert abs(w[t].sum() - 1.0) < 1e-12


def test_softmax_k_equals_E_is_full_softmax():
    lg = _rand_logits(11, 3, 16)
    ids, w = route.softmax_topk(lg, 16)
    for t in range(3):
        assert sorted(ids[t].tolist()) == list(range(16))
        np.testing.assert_allclose(w[t], softmax(lg[t].astype(np.float64))[ids[t]], rtol=1e-12)


def test_softmax_ties_go_to_lower_index():
    lg = np.array([[0.5, 2.0, 2.0, 1.0, 2.0]], dtype=np.float32)
    ids, w = route.softmax_topk(lg, 2)
    assert ids[0].tolist() == [1, 2]
    np.testing.assert_allclose(w[0], [0.5, 0.5])


def _group_score_brute(s_group):
    return max(s_group[a] + s_group[b] for a, b in itertools.combinations(range(len(s_group)), 2))


@pytest.mark.parametrize("seed", range(5))
def test_sigmoid_group_brute_force(seed):
    E, n_group, topk_group, k, scale = 16, 4, 2, 3, 2.5
    gs = E // n_group
    lg = _rand_logits(100 + seed, 8, E)
    ids, w = route.sigmoid_group(lg, k, n_group, topk_group, scale)
    for t in range(lg.shape[0]):
        s = expit(lg[t].astype(np.float64))
        scores = [_group_score_brute(s[g * gs:(g + 1) * gs]) for g in range(n_group)]
        kept = max(itertools.combinations(range(n_group), topk_group),
                   key=lambda c: sum(scores[g] for g in c))
        cand = [e for g in kept for e in range(g * gs, (g + 1) * gs)]
        best = max(itertools.combinations(cand, k), key=lambda c: sum(float(lg[t, i]) for i in c))
        assert set(ids[t].tolist()) == set(best)
        assert all(lg[t, ids[t, i]] >= lg[t, ids[t, i + 1]] for i in range(k - 1))
        np.testing.assert_allclose(w[t], s[ids[t]] / s[ids[t]].sum() * scale, rtol=1e-12)
        assert abs(w[t].sum() - scale) < 1e-12


def test_sigmoid_group_all_groups_is_plain_sigmoid_topk():
    lg = _rand_logits(7, 5, 32)
    ids, w = route.sigmoid_group(lg, 4, 8, 8, 1.0)
    for t in range(5):
        order = np.argsort(-lg[t], kind="stable")[:4]
        assert ids[t].tolist() == order.tolist()
        s = expit(lg[t].astype(np.float64))[order]
        np.testing.assert_allclose(w[t], s / s.sum(), rtol=1e-12)


def test_sigmoid_group_excludes_strong_expert_of_weak_group():
    # group 0 holds the single best logit, but its second best is poor, so its
    # top-2 sum loses to groups 1 and 2, and expert 0 must not be selected
    lg = np.full((1, 12), -6.0, dtype=np.float32)
    lg[0, 0] = 5.0                         # group 0: 5, -6 ...
    lg[0, 4:6] = [2.0, 1.9]                # group 1
    lg[0, 8:10] = [1.8, 1.7]               # group 2
    ids, _ = route.sigmoid_group(lg, 2, 3, 2, 1.0)
    assert ids[0].tolist() == [4, 5]


def test_router_logits_is_x_times_wr_transpose():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 8))
    wr = rng.standard_normal((5, 8))
    lg = route.router_logits(x, wr)
    for t in range(3):
        for e in range(5):
            assert abs(lg[t, e] - sum(x[t, h] * wr[e, h] for h in range(8))) < 1e-12
