"""Seeded activations and router-logit traces for the synthetic workloads.

Decode traces imitate the routing locality the FreeToken pages rely on (the
digest's "Results" and the English page's "Semantic-Aware Expert Caching":
consecutive tokens reuse most of their experts).  Per layer a random
permutation assigns Zipf popularity p(rank r) ~ r**-alpha; per step each of the
previous step's targets is kept with probability ``keep_prob`` and the set is
refilled by popularity sampling without replacement.  Target logits are
3 + N(0, 0.25); every other logit is N(-2, 0.5) clipped to at most -1, so the
top-k of every token is exactly its target set.

For grouped (sigmoid-group) routing the target set of a token spans at most
``topk_group`` groups of E / n_group consecutive experts.

Prefill logits are i.i.d. N(0, 1) (near-uniform routing).  Activations are
bf16-rounded N(0, 1); decode draws are independent per (step, layer).

Everything here is input generation only; none of the layer's arithmetic.
"""
from __future__ import annotations

import numpy as np

from .configs import ROUTE_SIGMOID_GROUP, Workload, seed
from .experts import bf16_bits_to_f32, f32_to_bf16_bits


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def bf16_normal(rng: np.random.Generator, shape) -> np.ndarray:
    """bf16 bits of N(0, 1) draws."""
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def decode_x(w: Workload, step: int, layer: int) -> np.ndarray:
    """Activations of one decode layer call, bf16 bits [T, H]."""
    return bf16_normal(_rng(seed(w.cid, 1), step, layer), (w.t_decode, w.hidden))


def prefill_x(w: Workload) -> np.ndarray:
    return bf16_normal(_rng(seed(w.cid, 1), 0xFFFF), (w.t_prefill, w.hidden))


def prefill_logits(w: Workload) -> np.ndarray:
    return _rng(seed(w.cid, 2), 0xFFFF).standard_normal(
        (w.t_prefill, w.n_experts), dtype=np.float32)


def prefill_x_layer(w: Workload, layer: int) -> np.ndarray:
    """Activations of one layer of a multi-layer prefill, bf16 bits [T, H]
    (independent per layer, like the decode draws)."""
    return bf16_normal(_rng(seed(w.cid, 1), 0xFFFE, layer), (w.t_prefill, w.hidden))


def prefill_logits_layer(w: Workload, layer: int) -> np.ndarray:
    return _rng(seed(w.cid, 2), 0xFFFE, layer).standard_normal(
        (w.t_prefill, w.n_experts), dtype=np.float32)


def tiny_inputs(w: Workload):
    """x bf16 bits [T, H] and router weights fp32 N(0, 0.02) [E, H]."""
    x = bf16_normal(_rng(seed(w.cid, 1)), (w.t_decode, w.hidden))
    wr = (_rng(seed(w.cid, 0), 7).standard_normal((w.n_experts, w.hidden)) * 0.02)
    return x, wr.astype(np.float32)


class DecodeTrace:
    """Router logits [steps, layers, T, E] fp32 for a decode workload."""

    def __init__(self, w: Workload, steps: int | None = None):
        self.w = w
        self.steps = w.steps if steps is None else steps
        rng = _rng(seed(w.cid, 2))
        E, L, T, k = w.n_experts, w.n_layers, w.t_decode, w.top_k
        ranks = np.arange(1, E + 1, dtype=np.float64)
        pop = ranks ** (-w.zipf_alpha)
        pop /= pop.sum()
        self.popularity = np.zeros((L, E))
        for l in range(L):
            self.popularity[l, rng.permutation(E)] = pop
        self.logits = np.empty((self.steps, L, T, E), dtype=np.float32)
        self.targets = np.empty((self.steps, L, T, k), dtype=np.int32)
        gsize = E // max(w.n_group, 1)
        grouped = w.route == ROUTE_SIGMOID_GROUP
        prev = [[None] * T for _ in range(L)]
        for s in range(self.steps):
            for l in range(L):
                for t in range(T):
                    keep = []
                    if prev[l][t] is not None:
                        keep = [e for e in prev[l][t] if rng.random() < w.keep_prob]
                    tgt = self._refill(rng, l, keep, k, gsize if grouped else 0, w.topk_group)
                    prev[l][t] = tgt
                    self.targets[s, l, t] = np.sort(np.asarray(tgt, dtype=np.int32))
                self.logits[s, l] = self._logits(rng, self.targets[s, l], E, k)

    def _refill(self, rng, l, keep, k, gsize, max_groups):
        chosen = list(keep)
        p = self.popularity[l]
        # popularity sampling without replacement through Gumbel keys, in key order
        keys = np.log(p) + rng.gumbel(size=p.size)
        for e in np.argsort(-keys, kind="stable"):
            if len(chosen) == k:
                break
            e = int(e)
            if e in chosen:
                continue
            if gsize:
                groups = {c // gsize for c in chosen}
                if e // gsize not in groups and len(groups) >= max_groups:
                    continue
            chosen.append(e)
        return chosen

    @staticmethod
    def _logits(rng, targets, E, k):
        T = targets.shape[0]
        while True:
            lg = np.minimum(rng.normal(-2.0, 0.5, size=(T, E)), -1.0).astype(np.float32)
            for t in range(T):
                lg[t, targets[t]] = (3.0 + rng.normal(0.0, 0.25, size=k)).astype(np.float32)
            srt = np.sort(lg, axis=1)[:, ::-1]
            if np.all(srt[:, k - 1] - srt[:, k] >= 0.5):
                return lg


def x_as_f32(x_bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(x_bits)
