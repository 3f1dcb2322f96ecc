"""A textbook LRU over ``collections.OrderedDict``, independent of ``cache``.

It pins ``cache.CacheSim``: choosing the K oldest slots once and consuming the
first q of them [FT-en, Elastic Memory Management] must equal q one-at-a-time
LRU evictions that skip entries touched in the same call, whenever q <= K.

Model: an ordered dict of slot -> content, oldest first.  It starts with every
slot empty, in ascending slot order.  A layer call looks its experts up, then
evicts from the front, skipping slots this call touched, and finally moves every
touched slot to the back in ascending slot order (entries touched in one call
share one timestamp and break the tie by slot).
"""
from __future__ import annotations

from collections import OrderedDict


class OrderedLRU:
    def __init__(self, n_slots: int, n_experts: int):
        self.E = n_experts
        self.order: "OrderedDict[int, int | None]" = OrderedDict((s, None) for s in range(n_slots))
        self.where: dict[int, int] = {}        # global expert id -> slot

    def call(self, layer: int, ids, K: int, q: int):
        want = sorted({layer * self.E + int(e) for e in ids})
        hits = {g: self.where[g] for g in want if g in self.where}
        misses = [g for g in want if g not in self.where]
        touched = set(hits.values())
        untouched = [s for s in self.order if s not in touched]
        victims = untouched[:K]
        n_fill = min(q, len(misses), len(victims))
        for i in range(n_fill):
            s = victims[i]
            old = self.order[s]
            if old is not None:
                del self.where[old]
            self.order[s] = misses[i]
            self.where[misses[i]] = s
            touched.add(s)
        for s in sorted(touched):
            self.order.move_to_end(s)
        return {
            "hit_expert": [g - layer * self.E for g in sorted(hits)],
            "fill_expert": [g - layer * self.E for g in misses[:n_fill]],
            "fill_slot": victims[:n_fill],
            "inplace": [g - layer * self.E for g in misses[n_fill:]],
            "victims": victims,
        }

    def shrink(self, n_new: int) -> "OrderedLRU":
        """Keep the n_new most recent occupied slots, renumbered by old slot order."""
        occupied = [s for s, g in self.order.items() if g is not None]
        keep = set(occupied[max(0, len(occupied) - n_new):])
        renumber = {old: new for new, old in enumerate(sorted(keep))}
        out = OrderedLRU(n_new, self.E)
        out.moved = sorted(renumber.items())     # (old slot, new slot) of every kept entry
        out.order = OrderedDict((s, None) for s in range(len(keep), n_new))
        for old in occupied:
            if old in keep:
                out.order[renumber[old]] = self.order[old]
                out.where[self.order[old]] = renumber[old]
        return out

    def table(self):
        return dict(self.where)
