"""Helpers shared by the GPU parity tests (imported lazily, safe on CPU)."""
from __future__ import annotations

import sys

import numpy as np

from workloads import configs as C
from workloads import experts as wx

# parity tolerances for the layer output (relative L2 and absolute)
REL_L2 = 1e-2
MAX_ABS = 2e-2


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def desc_of(w: C.Workload):
    import moe_expert_layer_02_amd as m
    return m.LayerDesc(w.hidden, w.inter, w.n_experts, w.top_k, w.route, w.n_group,
                       w.topk_group, w.route_scale, w.wfmt)


def packer(desc):
    """The library's canonical -> device layout conversion, as a pack(src, dst, n) callable."""
    import moe_expert_layer_02_amd as m
    return lambda src, dst, n: m.pack_experts(desc, src, dst, n)


def check_close(got, want, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = got - want
    rel = np.linalg.norm(err) / max(np.linalg.norm(want), 1e-30)
    mx = np.abs(err).max() if err.size else 0.0
    say(f"{what}: rel_l2={rel:.3e} max_abs={mx:.3e} (|ref| max {np.abs(want).max():.3e})")
    assert rel <= REL_L2, f"{what}: rel L2 {rel:.3e} > {REL_L2}"
    assert mx <= MAX_ABS, f"{what}: max abs {mx:.3e} > {MAX_ABS}"
    return rel, mx


class BlobSource:
    """CPU regeneration of expert bytes (independent of the GPU producer)."""

    def __init__(self, w: C.Workload, seed: int | None = None):
        self.w = w
        self.seed = C.seed(w.cid, 0) if seed is None else seed
        self.cache = {}

    def __call__(self, layer: int, e: int):
        g = layer * self.w.n_experts + e
        if g not in self.cache:
            self.cache[g] = wx.expert_blob(self.seed, g, self.w.wfmt, self.w.hidden, self.w.inter)
        return self.cache[g]


def oracle_layer(x, ids, w, blob, wfmt, H, I, tokens=None, workers=8, mx=False):
    """``ffn.moe_layer`` for the given tokens, its distinct experts split into
    disjoint groups evaluated in parallel threads.

    A token's output is the sum over its routed slots of w * y, so it equals
    the sum of the groups' partial outputs, each of which keeps the slots routed
    to its own experts (the others get weight 0 and point at one of the group's
    experts, so no other expert is dequantised).  NumPy releases the GIL in the
    dequantisation and the products, so the groups run concurrently.
    mx=True evaluates ``ffn.moe_layer_mx8`` instead (MXFP4 experts, MX
    activations): its x is quantised per token and h per pair, so the same
    split holds.
    """
    from concurrent.futures import ThreadPoolExecutor
    from oracle import ffn as offn
    ids = np.asarray(ids)
    w = np.asarray(w, dtype=np.float64)
    x = np.asarray(x)
    toks = np.arange(ids.shape[0]) if tokens is None else np.asarray(tokens)
    sid, sw, sx = ids[toks], w[toks], x[toks]
    experts = sorted({int(e) for e in sid.ravel()})
    n = max(1, min(workers, len(experts)))
    groups = [experts[i::n] for i in range(n)]

    def part(g):
        inside = np.isin(sid, g)
        gid, gw = np.where(inside, sid, g[0]), np.where(inside, sw, 0.0)
        if mx:
            return offn.moe_layer_mx8(sx, gid, gw, blob, H, I)
        return offn.moe_layer(sx, gid, gw, blob, wfmt, H, I)

    if n == 1:
        return part(groups[0])
    with ThreadPoolExecutor(n) as ex:
        return sum(ex.map(part, groups))


class ParityLog:
    """Collects float parity checks and reports the worst of them."""

    def __init__(self, what):
        self.what, self.worst_rel, self.worst_abs, self.n = what, 0.0, 0.0, 0

    def check(self, got, want, label):
        rel, mx = check_close(got, want, f"{self.what} {label}")
        self.worst_rel, self.worst_abs = max(self.worst_rel, rel), max(self.worst_abs, mx)
        self.n += 1

    def report(self):
        say(f"{self.what}: {self.n} float checks, worst rel_l2={self.worst_rel:.3e} "
            f"max_abs={self.worst_abs:.3e}")
