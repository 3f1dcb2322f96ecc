"""The expert cache's integer path, as a plain simulator.

What it follows:

* [FT-zh, Core method; FT-en, System Architecture] The full expert pool is
  the source of truth; a cache of N slots shared by every MoE layer holds the
  complete tensors of one (layer, expert) per slot.  The cache only changes
  speed, never results.
* [FT-zh, Core method and Method steps] Per layer call, on the device and with
  no host involvement: deduplicate the routed ids, classify them against the
  slot table into hits H and misses M, split the m = |M| misses into a fill set
  F of q experts copied into the cache and an in-place set C computed from the
  pool, pick K LRU victims with a single scan of the slot timestamps, and
  batch-copy F into the first q victims.
* [FT-zh, Core method] q* = m * B_P / B_H (the two bandwidths); it reduces to
  pure fill (q = m) when the two are equal.  [FT-en, Semantic-Aware Expert
  Caching] rounds 1.5 up to 2, so q is m * B_P / B_H rounded to nearest.
* [FT-en, Semantic-Aware Expert Caching] recency changes only when the router
  selects an expert.
* [FT-en, Elastic Memory Management] the single scan returns the K oldest
  slots; the miss path consumes the first q of them; the reused slots take the
  current step as their timestamp.  The slot budget is floor(budget / slot
  size), and a smaller budget evicts the excess slots at a safe point.

Readings (the pages leave these open):

* tick = step * L + layer + 1, one global counter per layer call, so recency is
  totally ordered across layers; 0 marks a never-used slot.
* Only slots with ts < tick are eligible, so this call's hits are never evicted;
  victims are the K smallest (ts, slot) pairs, ascending.
* F is the first q misses in ascending expert id; F[i] goes to victim i;
  q_eff = min(q, number of victims); the remaining misses form C.
* Rebuild keeps the ``n_new`` occupied slots that come last in the same
  (ts, slot) order, packs them into slots 0.. in ascending old-slot order and
  keeps their timestamps.
"""
from __future__ import annotations

import numpy as np


def q_split(m: int, q_num: int, q_den: int) -> int:
    """q = min(m, round(m * q_num / q_den)), halves rounded up, in integers."""
    return min(m, (2 * q_num * m + q_den) // (2 * q_den))


def slots_for_budget(budget_bytes: int, slot_bytes: int) -> int:
    """Number of cache slots a memory budget buys."""
    return budget_bytes // slot_bytes


class CacheSim:
    """Slot table [L*E], slot owner [N] and slot timestamps [N]."""

    def __init__(self, n_slots: int, n_layers: int, n_experts: int):
        self.N, self.L, self.E = n_slots, n_layers, n_experts
        self.table = np.full(n_layers * n_experts, -1, dtype=np.int32)
        self.owner = np.full(n_slots, -1, dtype=np.int32)
        self.ts = np.zeros(n_slots, dtype=np.int64)

    def copy(self) -> "CacheSim":
        c = CacheSim(self.N, self.L, self.E)
        c.table[:] = self.table
        c.owner[:] = self.owner
        c.ts[:] = self.ts
        return c

    def classify_evict(self, layer: int, tick: int, ids, K: int, q_num: int = 1, q_den: int = 1):
        """One layer call.  Returns a dict of the call's lists and counts."""
        base = layer * self.E
        uniq = sorted({int(e) for e in np.asarray(ids).ravel()})
        hit_e, hit_s, miss = [], [], []
        for e in uniq:
            s = int(self.table[base + e])
            if s >= 0:
                hit_e.append(e)
                hit_s.append(s)
            else:
                miss.append(e)
        for s in hit_s:                       # recency moves only on a router selection
            self.ts[s] = tick
        q = q_split(len(miss), q_num, q_den)
        # one scan over every slot's timestamp: the K oldest eligible slots
        eligible = np.nonzero(self.ts < tick)[0]              # ascending slot ids
        order = np.argsort(self.ts[eligible], kind="stable")    # by ts, then slot
        victims = [int(s) for s in eligible[order][:K]]
        q_eff = min(q, len(victims))
        fill_e = miss[:q_eff]
        fill_s = victims[:q_eff]
        for e, v in zip(fill_e, fill_s):
            old = int(self.owner[v])
            if old >= 0:
                self.table[old] = -1
            self.table[base + e] = v
            self.owner[v] = base + e
            self.ts[v] = tick
        return {
            "uniq": uniq, "hit_expert": hit_e, "hit_slot": hit_s, "miss": miss,
            "fill_expert": fill_e, "fill_slot": fill_s, "inplace": miss[q_eff:],
            "victims": victims,
            "counts": [len(uniq), len(hit_e), len(miss), q_eff, len(miss) - q_eff, len(victims)],
        }

    def rebuild(self, n_new: int) -> "CacheSim":
        """A cache of n_new slots holding the most recent entries of this one."""
        occ = [(int(self.ts[s]), s) for s in range(self.N) if self.owner[s] >= 0]
        occ.sort()
        kept = sorted(s for _, s in occ[max(0, len(occ) - n_new):])
        new = CacheSim(n_new, self.L, self.E)
        for new_slot, old_slot in enumerate(kept):
            g = int(self.owner[old_slot])
            new.owner[new_slot] = g
            new.ts[new_slot] = self.ts[old_slot]
            new.table[g] = new_slot
        return new

    def moves_of_rebuild(self, n_new: int):
        """(old slot, new slot) pairs whose bytes a rebuild copies, read off the
        rebuilt cache: new slot n holds owner g, which sat in slot table[g] here."""
        new = self.rebuild(n_new)
        return [(int(self.table[g]), n) for n, g in enumerate(new.owner.tolist()) if g >= 0]
