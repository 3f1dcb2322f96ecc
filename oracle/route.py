"""Router: logits and the two routing families.

[Edge0, section 2 "MoE routing"]: production sparse MoE layers route each
token to k of E experts with one of two families.

* softmax-top-k: an exact softmax over the E logits, keep the k largest,
  renormalise over the kept ones.  Softmax is monotone in the logit, so the
  selection is taken on the float32 logit itself, and the renormalised weights
  equal exp(l_j - l_max) / sum over the kept set of exp(l - l_max).
* sigmoid-group: score every expert with a sigmoid; rank groups by the sum of
  each group's two best scores; keep the best ``topk_group`` groups; take the
  top-k experts inside them; weights are the kept raw sigmoid scores,
  renormalised and multiplied by a scale factor.

Readings where the page is silent: ties go to the lower index (expert or
group); a group is a block of E / n_group consecutive experts; no correction
bias; the group scores are formed in float64 from the float32 logits; inside the
kept groups experts are ranked by the float32 logit (the sigmoid is monotone);
the selected ids are listed in descending score order.
"""
from __future__ import annotations

import numpy as np


def router_logits(x: np.ndarray, w_router: np.ndarray, dtype=np.float64) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] * W_r[e, h]."""
    return np.asarray(x, dtype=dtype) @ np.asarray(w_router, dtype=dtype).T


def _descending(values: np.ndarray, candidates: np.ndarray) -> np.ndarray:
    """Candidates ordered by descending value, ties by ascending index."""
    cand = np.sort(np.asarray(candidates))
    order = np.argsort(-values[cand], kind="stable")
    return cand[order]


def softmax_topk(logits: np.ndarray, k: int):
    """ids int32 [T, k], weights float64 [T, k]."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        sel = _descending(lg[t], np.arange(E))[:k]
        l = lg[t, sel].astype(np.float64)
        p = np.exp(l - l.max())
        ids[t] = sel
        w[t] = p / p.sum()
    return ids, w


def sigmoid(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def sigmoid_group(logits: np.ndarray, k: int, n_group: int, topk_group: int, scale: float):
    """ids int32 [T, k], weights float64 [T, k]."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    gsize = E // n_group
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        s = sigmoid(lg[t])
        gscore = np.empty(n_group, dtype=np.float64)
        for g in range(n_group):
            best2 = np.sort(s[g * gsize:(g + 1) * gsize])[::-1][:2]
            gscore[g] = best2[0] + best2[1]
        kept = _descending(gscore, np.arange(n_group))[:topk_group]
        cand = np.concatenate([np.arange(g * gsize, (g + 1) * gsize) for g in kept])
        sel = _descending(lg[t], cand)[:k]
        ids[t] = sel
        w[t] = s[sel] / s[sel].sum() * scale
    return ids, w


def route(logits: np.ndarray, k: int, kind: int, n_group: int = 1, topk_group: int = 1,
          scale: float = 1.0):
    if kind == 0:
        return softmax_topk(logits, k)
    if kind == 1:
        return sigmoid_group(logits, k, n_group, topk_group, scale)
    raise ValueError(kind)
