"""The decode-layer calls on the GPU, in both orders the library offers:
"fused" (route + classify_evict in one kernel, or the whole call in one launch
for small calls, then the expert FFN with fill-through) and "split" (route +
plan, the FFN reading misses from the pool, and the LRU update + fill copy on a
second stream that the next layer waits for).

Every call of decode traces is checked bit-exact against the oracle's
simulator on the integer outputs; layer outputs are checked against the oracle
on whole steps (every layer) for the Qwen-like trace and on every token of
several calls for the DS-like ones (calls with in-place experts, the cold
start, and the calls right after the stress workload's budget shrink); every
cache slot holds its owner's pool bytes afterwards; the workspace's error word
stays clear after every step.  A run with the tick near 2^30 takes the victim
scan's 64-bit key path.  A whole decode step captured as a graph and replayed
is checked the same way against the oracle."""
import numpy as np
import pytest

from oracle import cache as ocache
from oracle import route as oroute
from workloads import configs as C
from workloads import experts as wx
from workloads import traces as tr

from gpu_common import BlobSource, ParityLog, desc_of, oracle_layer, packer, say

pytestmark = pytest.mark.gpu

WIDE_TICK = 1 << 30     # tick << log2(N) no longer fits 32 bits: 64-bit victim keys


def _x_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


class LayerRunner:
    def __init__(self, w, n_slots, pool, mode="fused", tick0=0):
        import torch
        import moe_expert_layer_02_amd as m
        self.m, self.torch, self.w, self.mode, self.tick0 = m, torch, w, mode, tick0
        self.side = torch.cuda.Stream()
        self.planned = [torch.cuda.Event() for _ in range(w.n_layers)]
        self.desc = desc_of(w)
        self.S = wx.expert_bytes(w.wfmt, w.hidden, w.inter)
        self.cache = m.DeviceCache(n_slots, w.n_layers, w.n_experts, self.S)
        self.pool = pool
        self.K = min(w.t_decode * w.top_k, w.n_experts, n_slots)
        self.policy = m.EvictPolicy(self.K, w.q_num, w.q_den)
        self.cap = max(self.K, min(w.t_decode * w.top_k, w.n_experts))
        L, T = w.n_layers, w.t_decode
        self.lists = [m.DeviceClassifyOut(self.cap) for _ in range(L)]
        self.ids = torch.empty((L, T, w.top_k), dtype=torch.int32, device="cuda")
        self.wt = torch.empty((L, T, w.top_k), dtype=torch.float32, device="cuda")
        self.out = torch.empty((L, T, w.hidden), dtype=torch.float32, device="cuda")
        self.ws = torch.zeros(m.workspace_bytes(self.desc, T, m.MODE_DECODE), dtype=torch.uint8,
                              device="cuda")
        self.tick = torch.zeros(1, dtype=torch.int64, device="cuda")
        self.logits = torch.empty((L, T, w.n_experts), dtype=torch.float32, device="cuda")
        self.x = torch.empty((L, T, w.hidden), dtype=torch.bfloat16, device="cuda")

    def tick_of(self, step, layer):
        return self.tick0 + step * self.w.n_layers + layer + 1

    def stage(self, step, logits_np, xs):
        self.logits.copy_(self.torch.from_numpy(logits_np))
        self.x.copy_(xs)
        self.tick.fill_(self.tick0 + step * self.w.n_layers)

    def rebuild(self, n_new):
        """Elastic budget change at a step boundary: a new cache of n_new slots."""
        m = self.m
        new = m.DeviceCache(n_new, self.w.n_layers, self.w.n_experts, self.S)
        m.cache_rebuild(self.cache, new)
        self.cache = new
        self.K = min(self.w.t_decode * self.w.top_k, self.w.n_experts, n_new)
        self.policy = m.EvictPolicy(self.K, self.w.q_num, self.w.q_den)
        assert self.K <= self.cap

    def step(self):
        m = self.m
        main = self.torch.cuda.current_stream()
        if self.mode == "split":
            self.side.wait_stream(main)   # staged inputs
        for l in range(self.w.n_layers):
            if self.mode == "fused":
                m.decode_layer(self.desc, self.cache, self.pool, l, self.tick, l + 1,
                               self.logits[l], self.x[l], self.policy, self.ids[l], self.wt[l],
                               self.lists[l], self.out[l], self.ws)
                continue
            main.wait_stream(self.side)   # the previous layer's slot update and fill
            m.route_plan(self.desc, self.cache, l, self.logits[l], self.ids[l], self.wt[l],
                         self.lists[l])
            self.planned[l].record(main)
            m.expert_ffn_decode(self.desc, self.x[l], self.ids[l], self.wt[l], self.cache,
                                self.pool, l, self.lists[l], self.out[l], self.ws)
            self.side.wait_event(self.planned[l])
            m.evict_fill(self.desc, self.cache, self.pool, l, self.tick, l + 1, self.ids[l],
                         self.policy, self.lists[l], stream=self.side)
        if self.mode == "split":
            main.wait_stream(self.side)


def _xs(w, s):
    import torch
    return torch.stack([_x_dev(tr.decode_x(w, s, l)) for l in range(w.n_layers)])


def _check_ints(run, sim, s, w, logits):
    """Every layer call of step s bit-exact against the simulator; returns the
    oracle's (ids, weights, call dict) per layer."""
    routed = []
    for l in range(w.n_layers):
        rid, rw = oroute.route(logits[l], w.top_k, w.route, w.n_group, w.topk_group,
                               w.route_scale)
        exp = sim.classify_evict(l, run.tick_of(s, l), rid, run.K, w.q_num, w.q_den)
        got = run.lists[l].host()
        assert got["counts"] == exp["counts"], (s, l, got["counts"], exp["counts"])
        for key in ("uniq", "hit_expert", "hit_slot", "miss", "fill_expert", "fill_slot",
                    "inplace", "victims"):
            assert got[key] == exp[key], (s, l, key)
        assert np.array_equal(run.ids[l].cpu().numpy(), rid), (s, l)
        routed.append((rid, rw, exp))
    return routed


def _check_cache_state(run, sim, pool):
    import torch
    assert np.array_equal(run.cache.table.cpu().numpy(), sim.table)
    assert np.array_equal(run.cache.owner.cpu().numpy(), sim.owner)
    assert np.array_equal(run.cache.ts.cpu().numpy(), sim.ts)
    S = run.S
    owner = run.cache.owner.cpu().numpy()
    data, pv = run.cache.data.view(-1, S), pool.view(-1, S)
    occ = np.nonzero(owner >= 0)[0]
    for i in range(0, len(occ), 64):
        sl = torch.from_numpy(occ[i:i + 64]).cuda()
        ow = torch.from_numpy(owner[occ[i:i + 64]].astype(np.int64)).cuda()
        assert torch.equal(data.index_select(0, sl), pv.index_select(0, ow)), "slot bytes differ"
    return len(occ)


class Sampler:
    """Which calls' outputs to check against the oracle, decided while the
    trace runs (the outputs are overwritten by the next step)."""

    def __init__(self, steps_all_layers=(), calls=(), first_inplace=0, after_rebuild=(),
                 tokens=None):
        self.steps_all = set(steps_all_layers)
        self.calls = set(calls)
        self.first_inplace = first_inplace      # how many of the first in-place calls
        self.after_rebuild = set(after_rebuild)
        self.tokens = tokens
        self.jobs = []

    def pick(self, s, l, exp):
        if s in self.steps_all or (s, l) in self.calls or (s, l) in self.after_rebuild:
            return True
        if self.first_inplace and exp["counts"][4] > 0:
            self.first_inplace -= 1
            return True
        return False

    def take(self, run, s, routed):
        w = run.w
        toks = list(range(w.t_decode)) if self.tokens is None else self.tokens
        out = None
        for l, (rid, rw, exp) in enumerate(routed):
            if self.pick(s, l, exp):
                out = run.out.cpu().numpy() if out is None else out
                tag = f"call ({s},{l}) hits {exp['counts'][1]} fills {exp['counts'][3]} " \
                      f"in-place {exp['counts'][4]}"
                self.jobs.append((tag, l, tr.decode_x(w, s, l), rid, rw, toks, out[l][toks].copy()))

    def verify(self, w, src, what):
        log = ParityLog(what)
        for tag, l, xb, rid, rw, toks, got in self.jobs:
            want = oracle_layer(tr.x_as_f32(xb), rid, rw, lambda e, l=l: src(l, e), w.wfmt,
                                w.hidden, w.inter, tokens=toks)
            log.check(got, want, tag)
        log.report()
        assert log.n == len(self.jobs) and log.n > 0


# Small multi-token calls that take the one-launch whole-layer path (several
# routing wavefronts, several token columns in the down products), with caches
# small enough to evict every step: int4 + softmax-top-k, MXFP4 + sigmoid-group.
EXTRA = {
    6: C.Workload(cid=6, name="small_int4_t3", hidden=1024, inter=256, n_experts=32, top_k=4,
                  route=C.ROUTE_SOFTMAX_TOPK, wfmt=C.WFMT_INT4_G64, n_layers=4, n_slots=64,
                  t_decode=3, steps=40, zipf_alpha=1.1, keep_prob=0.5, q_num=2, q_den=3),
    7: C.Workload(cid=7, name="small_mxfp4_t2", hidden=2048, inter=256, n_experts=64, top_k=4,
                  route=C.ROUTE_SIGMOID_GROUP, n_group=8, topk_group=2, route_scale=2.5,
                  wfmt=C.WFMT_MXFP4, n_layers=4, n_slots=96, t_decode=2, steps=40,
                  zipf_alpha=1.0, keep_prob=0.6),
    # one token per call: the whole-layer launch publishes the plan as a record
    8: C.Workload(cid=8, name="small_mxfp4_sig_t1", hidden=2048, inter=256, n_experts=64, top_k=6,
                  route=C.ROUTE_SIGMOID_GROUP, n_group=8, topk_group=4, route_scale=2.5,
                  wfmt=C.WFMT_MXFP4, n_layers=4, n_slots=48, t_decode=1, steps=40,
                  zipf_alpha=1.0, keep_prob=0.6),
    9: C.Workload(cid=9, name="small_int4_t1_split", hidden=1024, inter=256, n_experts=32, top_k=8,
                  route=C.ROUTE_SOFTMAX_TOPK, wfmt=C.WFMT_INT4_G64, n_layers=4, n_slots=40,
                  t_decode=1, steps=40, zipf_alpha=1.1, keep_prob=0.5, q_num=1, q_den=2),
}


def _workload(cid):
    return C.ALL[cid] if cid in C.ALL else EXTRA[cid]


def _sampler(cid, steps, mode):
    w = _workload(cid)
    if cid == 2:      # every layer of a middle and the last step
        return Sampler(steps_all_layers=(steps // 2 - 1, steps - 1))
    if cid == 4:      # the cold start, the last call, two in between, the first in-place calls
        calls = [(0, 0), (steps - 1, w.n_layers - 1)]
        if mode == "fused":
            calls += [(5, 7), (steps // 2, 11)]
        return Sampler(calls=calls, first_inplace=1 if mode == "fused" else 0)
    if cid == 5:      # in-place calls, and the calls around the budget shrink when crossed
        after = ()
        if steps > w.shrink_step:
            s0 = w.shrink_step
            after = [(s0 - 1, w.n_layers - 1), (s0, 0), (s0, w.n_layers // 2), (steps - 1, w.n_layers - 1)]
        return Sampler(calls=[(steps - 1, w.n_layers - 1)], first_inplace=2, after_rebuild=after)
    return Sampler(calls=[(0, 0), (0, 1), (steps // 2, 2), (steps - 1, w.n_layers - 1)],
                   first_inplace=2)


CASES = [
    # (workload, steps, tick base, pool in pinned host memory)
    (2, 64, 0, False), (4, 24, 0, False), (5, 24, 0, False), (6, 40, 0, False), (7, 40, 0, False),
    (8, 40, 0, False), (9, 40, 0, False),
    (2, 16, WIDE_TICK, False), (9, 40, WIDE_TICK, False), (4, 8, WIDE_TICK, False),
    # the host tier: misses read (in place, or while filling) over PCIe from pinned memory
    (9, 40, 0, True), (7, 40, 0, True), (6, 40, 0, True),
]


def _run_decode_trace(cid, steps, mode, tick0, host_pool=False):
    import torch
    import moe_expert_layer_02_amd as m
    from workloads import gpu as wg
    w = _workload(cid)
    say(f"decode_layer trace {w.name} ({mode}): {steps} steps, tick base {tick0}, "
        f"pool in {'pinned host' if host_pool else 'device'} memory")
    trace = tr.DecodeTrace(w, steps)
    pool_dev = wg.make_pool(w, pack=packer(desc_of(w)))
    pool = pool_dev
    if host_pool:
        pool = torch.empty(pool_dev.numel(), dtype=torch.uint8, pin_memory=True)
        pool.copy_(pool_dev)
    run = LayerRunner(w, w.n_slots, pool, mode, tick0=tick0)
    sim = ocache.CacheSim(w.n_slots, w.n_layers, w.n_experts)
    sampler = _sampler(cid, steps, mode)
    for s in range(steps):
        if s == w.shrink_step:
            torch.cuda.synchronize()
            run.rebuild(w.shrink_slots)
            sim = sim.rebuild(w.shrink_slots)
            say(f"{w.name}: budget shrunk to {w.shrink_slots} slots at step {s}")
        xs = _xs(w, s)
        run.stage(s, trace.logits[s], xs)
        run.step()
        torch.cuda.synchronize()
        m.check_error(run.ws, what=f"{w.name} step {s}")
        routed = _check_ints(run, sim, s, w, trace.logits[s])
        sampler.take(run, s, routed)
        if s % 64 == 63:
            say(f"{w.name}: step {s + 1}/{steps}")
    n_occ = _check_cache_state(run, sim, pool_dev)
    say(f"{w.name}: {steps * w.n_layers} calls bit-exact, {n_occ} slots hold their pool bytes")
    sampler.verify(w, BlobSource(w), f"{w.name} ({mode})")


@pytest.mark.parametrize("mode", ["fused", "split"])
@pytest.mark.parametrize("cid,steps,tick0,host_pool", CASES)
def test_decode_layer_trace(cid, steps, tick0, host_pool, mode):
    _run_decode_trace(cid, steps, mode, tick0, host_pool)


@pytest.mark.timeout(900)
def test_decode_layer_stress_across_budget_shrink():
    """The stress workload's decode trace through its budget shrink (1024 -> 384
    slots at step 256) with the fused layer calls: every call bit-exact, the
    calls right before and after the shrink checked on every token."""
    w = C.DS_STRESS
    _run_decode_trace(5, w.shrink_step + 6, "fused", 0)


def test_decode_layer_workspace_header_left_zero():
    """Whole-layer calls of two shapes share one workspace, steps alternating: a
    one-token call (its plan travels as a 64-byte record in every plan-flag
    copy) and a three-token call (plain flags).  After every step the first
    65536 bytes, error word included, are zero again, and the outputs match
    the oracle on sampled calls."""
    import torch
    from workloads import gpu as wg
    ws_ = None
    runs = []
    for cid in (9, 6):
        w = EXTRA[cid]
        run = LayerRunner(w, w.n_slots, wg.make_pool(w, pack=packer(desc_of(w))), "fused")
        ws_ = run.ws if ws_ is None or run.ws.numel() > ws_.numel() else ws_
        runs.append((w, run, tr.DecodeTrace(w, 6), BlobSource(w)))
    for _, run, _, _ in runs:
        run.ws = ws_
    log = ParityLog("shared workspace")
    for s in range(6):
        for w, run, trace, src in runs:
            xs = _xs(w, s)
            run.stage(s, trace.logits[s], xs)
            run.step()
            torch.cuda.synchronize()
            assert int(ws_[:65536].count_nonzero()) == 0, (w.name, s)
            l = s % w.n_layers
            rid, rw = oroute.route(trace.logits[s, l], w.top_k, w.route, w.n_group,
                                   w.topk_group, w.route_scale)
            want = oracle_layer(tr.x_as_f32(tr.decode_x(w, s, l)), rid, rw,
                                lambda e: src(l, e), w.wfmt, w.hidden, w.inter)
            log.check(run.out[l].cpu().numpy(), want, f"{w.name} ({s},{l})")
    log.report()
    say("workspace header zero after every step, two shapes sharing it")


@pytest.mark.parametrize("mode", ["fused", "split"])
def test_decode_step_graph_replay_matches_oracle(mode):
    """A whole Qwen-like decode step (40 layer calls, a device-resident tick)
    captured once and replayed over six steps of the trace, with the inputs
    staged eagerly between replays: every replay's lists bit-exact against the
    simulator, ids against the oracle's routing, four layers' outputs per step
    against the oracle, and the final cache state and slot bytes."""
    import torch
    import moe_expert_layer_02_amd as m
    from workloads import gpu as wg
    w = C.QWEN_DECODE
    steps = 6
    trace = tr.DecodeTrace(w, steps)
    pool = wg.make_pool(w, pack=packer(desc_of(w)))
    # one eager step on a throwaway cache, so no kernel is launched for the
    # first time (occupancy query) while the graph is being captured
    warm = LayerRunner(w, w.n_slots, pool, mode)
    warm.stage(0, trace.logits[0], _xs(w, 0))
    warm.step()
    torch.cuda.synchronize()
    del warm
    graphed = LayerRunner(w, w.n_slots, pool, mode)
    graphed.stage(0, trace.logits[0], _xs(w, 0))
    torch.cuda.synchronize()
    snap = [t.clone() for t in (graphed.cache.table, graphed.cache.owner, graphed.cache.ts)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.step()
    torch.cuda.synchronize()
    # capturing records the launches without running them
    for a, b in zip(snap, (graphed.cache.table, graphed.cache.owner, graphed.cache.ts)):
        assert torch.equal(a, b)
    sim = ocache.CacheSim(w.n_slots, w.n_layers, w.n_experts)
    sampler = Sampler(calls=[(s, l) for s in range(steps) for l in (0, 13, 26, 39)])
    for s in range(steps):
        graphed.stage(s, trace.logits[s], _xs(w, s))
        g.replay()
        torch.cuda.synchronize()
        m.check_error(graphed.ws, what=f"replay {s}")
        routed = _check_ints(graphed, sim, s, w, trace.logits[s])
        sampler.take(graphed, s, routed)
        say(f"graph replay {s} ({mode}): {w.n_layers} calls bit-exact against the simulator")
    _check_cache_state(graphed, sim, pool)
    sampler.verify(w, BlobSource(w), f"graph replay ({mode})")
