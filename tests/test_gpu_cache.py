"""Cache integer-path parity on the GPU: every layer call of whole decode
traces (route -> classify_evict -> cache_fill) against the oracle's simulator,
bit-exact on every list and count and on the final slot table, owner and
timestamps; fill bytes checked against the pool; the mid-run budget shrink of
the cache-pressure workload through cache_rebuild."""
import numpy as np
import pytest

from oracle import cache as ocache
from oracle import route as oroute
from workloads import configs as C
from workloads import experts as wx
from workloads import traces as tr

from gpu_common import desc_of, say

pytestmark = pytest.mark.gpu

KEYS = ("uniq", "hit_expert", "hit_slot", "miss", "fill_expert", "fill_slot", "inplace", "victims")


class TraceRunner:
    """Drives the GPU path for a decode trace, keeping every call's lists on device."""

    def __init__(self, w, n_slots, pool, steps):
        import torch
        import moe_expert_layer_02_amd as m
        self.m, self.torch, self.w = m, torch, w
        self.S = wx.expert_bytes(w.wfmt, w.hidden, w.inter)
        self.cache = m.DeviceCache(n_slots, w.n_layers, w.n_experts, self.S,
                                   with_data=pool is not None)
        self.pool = pool
        self.K = w.victims_k
        self.cap = max(self.K, min(w.t_decode * w.top_k, w.n_experts))
        n_calls = steps * w.n_layers
        self.lists = torch.full((n_calls, len(KEYS), self.cap), -1, dtype=torch.int32, device="cuda")
        self.counts = torch.zeros((n_calls, 6), dtype=torch.int32, device="cuda")
        self.plan = torch.zeros((n_calls, self.cap, 4), dtype=torch.int32, device="cuda")
        self.pairs = torch.zeros((n_calls, w.t_decode * w.top_k), dtype=torch.int32,
                                 device="cuda")
        self.desc = desc_of(w)
        self.ids = torch.empty((w.t_decode, w.top_k), dtype=torch.int32, device="cuda")
        self.wt = torch.empty((w.t_decode, w.top_k), dtype=torch.float32, device="cuda")

    def out_struct(self, call):
        m = self.m
        o = m.DeviceClassifyOut.__new__(m.DeviceClassifyOut)
        o.capacity = self.cap
        o.buf = self.lists[call]
        o.counts = self.counts[call]
        o.plan = self.plan[call]
        o.pairs = self.pairs[call]
        o.struct = m.ClassifyOut(*[o.buf[i].data_ptr() for i in range(len(KEYS))],
                                 o.counts.data_ptr(), self.cap, o.plan.data_ptr(),
                                 o.pairs.data_ptr(), self.pairs.shape[1])
        return o

    def call(self, call_idx, layer, tick, logits_np, policy):
        m, torch = self.m, self.torch
        lg = torch.from_numpy(np.ascontiguousarray(logits_np)).cuda()
        m.route(self.desc, lg, self.ids, self.wt)
        o = self.out_struct(call_idx)
        m.classify_evict(self.cache, layer, tick, self.ids, policy, o)
        if self.pool is not None:
            m.cache_fill(self.cache, self.pool, layer, o, self.K)

    def host_call(self, call_idx, lists, counts):
        c = counts[call_idx].tolist()
        n = {"uniq": c[0], "hit_expert": c[1], "hit_slot": c[1], "miss": c[2], "fill_expert": c[3],
             "fill_slot": c[3], "inplace": c[4], "victims": c[5]}
        return {k: lists[call_idx, i, :n[k]].tolist() for i, k in enumerate(KEYS)}, c


def _run_trace(w, steps, with_pool, shrink_step=-1, shrink_slots=0, tick0=0):
    import torch
    import moe_expert_layer_02_amd as m
    from workloads import gpu as wg
    say(f"cache trace {w.name}: steps={steps} L={w.n_layers} N={w.n_slots} pool={with_pool} "
        f"tick base {tick0}")
    trace = tr.DecodeTrace(w, steps)
    pool = wg.make_pool(w) if with_pool else None
    runner = TraceRunner(w, w.n_slots, pool, steps)
    sim = ocache.CacheSim(w.n_slots, w.n_layers, w.n_experts)
    policy = m.EvictPolicy(runner.K, w.q_num, w.q_den)
    expected = []
    routed = []
    for s in range(steps):
        if s == shrink_step:
            torch.cuda.synchronize()
            new = m.DeviceCache(shrink_slots, w.n_layers, w.n_experts, runner.S,
                                with_data=with_pool)
            m.cache_rebuild(runner.cache, new)
            torch.cuda.synchronize()
            sim = sim.rebuild(shrink_slots)
            assert np.array_equal(new.table.cpu().numpy(), sim.table)
            assert np.array_equal(new.owner.cpu().numpy(), sim.owner)
            assert np.array_equal(new.ts.cpu().numpy(), sim.ts)
            runner.cache = new
            runner.K = min(w.t_decode * w.top_k, w.n_experts, shrink_slots)
            policy = m.EvictPolicy(runner.K, w.q_num, w.q_den)
            say(f"rebuilt to {shrink_slots} slots at step {s}")
        if s % 64 == 0:
            say(f"{w.name}: step {s}/{steps}")
        for l in range(w.n_layers):
            call = s * w.n_layers + l
            tick = tick0 + call + 1
            runner.call(call, l, tick, trace.logits[s, l], policy)
            ids, _ = oroute.route(trace.logits[s, l], w.top_k, w.route, w.n_group, w.topk_group,
                                  w.route_scale)
            expected.append(sim.classify_evict(l, tick, ids, runner.K, w.q_num, w.q_den))
            routed.append(ids.ravel())
    torch.cuda.synchronize()
    lists = runner.lists.cpu().numpy()
    counts = runner.counts.cpu().numpy()
    plans = runner.plan.cpu().numpy()
    pairs = runner.pairs.cpu().numpy()
    for call, exp in enumerate(expected):
        got, c = runner.host_call(call, lists, counts)
        assert c == exp["counts"], (call, c, exp["counts"])
        for k in KEYS:
            assert got[k] == exp[k], (call, k, got[k], exp[k])
        _check_plan(exp, plans[call], pairs[call], routed[call])
    assert np.array_equal(runner.cache.table.cpu().numpy(), sim.table)
    assert np.array_equal(runner.cache.owner.cpu().numpy(), sim.owner)
    assert np.array_equal(runner.cache.ts.cpu().numpy(), sim.ts)
    n_miss = sum(e["counts"][2] for e in expected)
    n_u = sum(e["counts"][0] for e in expected)
    say(f"{w.name}: {len(expected)} calls bit-exact; miss rate {n_miss / max(n_u, 1):.3f}")
    if with_pool:
        _check_slot_bytes(runner, pool, w)
    return runner, pool


def _check_plan(exp, plan, pairs, ids):
    """plan[u] = (slot after the call or -1, filled now, first pair, pair count)."""
    slot_of = dict(zip(exp["hit_expert"], exp["hit_slot"]))
    fill_of = dict(zip(exp["fill_expert"], exp["fill_slot"]))
    begin = 0
    for u, e in enumerate(exp["uniq"]):
        want_slot = slot_of.get(e, fill_of.get(e, -1))
        want = [want_slot, 1 if e in fill_of else 0, begin, int((ids == e).sum())]
        assert plan[u].tolist() == want, (u, e, plan[u].tolist(), want)
        grp = sorted(pairs[begin:begin + want[3]].tolist())
        assert grp == [i for i in range(len(ids)) if ids[i] == e]
        begin += want[3]


def _check_slot_bytes(runner, pool, w):
    import torch
    S = runner.S
    owner = runner.cache.owner.cpu().numpy()
    data = runner.cache.data.view(-1, S)
    pv = pool.view(-1, S)
    occ = np.nonzero(owner >= 0)[0]
    for i in range(0, len(occ), 64):
        sl = torch.from_numpy(occ[i:i + 64]).cuda()
        ow = torch.from_numpy(owner[occ[i:i + 64]].astype(np.int64)).cuda()
        assert torch.equal(data.index_select(0, sl), pv.index_select(0, ow)), "slot bytes differ"
    say(f"{len(occ)} occupied slots hold their owner's pool bytes")


def test_synth_pool_matches_cpu_generator():
    import torch
    from workloads import gpu as wg
    for w in (C.TINY, C.QWEN_DECODE, C.DS_DECODE):
        S = wx.expert_bytes(w.wfmt, w.hidden, w.inter)
        for g in (0, 7, w.n_layers * w.n_experts - 1):
            buf = torch.empty(S, dtype=torch.uint8, device="cuda")
            wg.fill_experts(buf, g, 1, w.wfmt, w.hidden, w.inter, C.seed(w.cid, 0))
            ref = wx.expert_blob(C.seed(w.cid, 0), g, w.wfmt, w.hidden, w.inter)
            assert np.array_equal(buf.cpu().numpy(), ref), (w.name, g)


def test_cache_trace_qwen_decode():
    _run_trace(C.QWEN_DECODE, C.QWEN_DECODE.steps, with_pool=True)


def test_cache_trace_ds_decode():
    _run_trace(C.DS_DECODE, C.DS_DECODE.steps, with_pool=True)


def test_cache_trace_stress_with_rebuild():
    w = C.DS_STRESS
    runner, pool = _run_trace(w, w.steps, with_pool=True, shrink_step=w.shrink_step,
                              shrink_slots=w.shrink_slots)


# Ticks near 2^30: (tick << log2 N) no longer fits 32 bits, so the victim scan
# ranks 64-bit keys (few victims: the Qwen-like K = 8 over 2048 slots; many:
# the DS-like K = 96 radix select over 1024 slots, and the stress run's rebuild).
WIDE_TICK = 1 << 30


def test_cache_trace_qwen_decode_wide_keys():
    _run_trace(C.QWEN_DECODE, 48, with_pool=False, tick0=WIDE_TICK)


def test_cache_trace_ds_decode_wide_keys():
    _run_trace(C.DS_DECODE, 32, with_pool=False, tick0=WIDE_TICK)


def test_cache_trace_stress_wide_keys_with_rebuild():
    w = C.DS_STRESS
    _run_trace(w, 40, with_pool=True, shrink_step=20, shrink_slots=w.shrink_slots,
               tick0=WIDE_TICK)


def test_classify_small_cache_every_path():
    """A tiny cache where victims run out, q splits and evictions cross layers."""
    import torch
    import moe_expert_layer_02_amd as m
    w = C.Workload(cid=95, name="tinycache", hidden=256, inter=128, n_experts=16, top_k=3,
                   route=0, n_layers=3, n_slots=5, t_decode=3, steps=40, zipf_alpha=0.8,
                   keep_prob=0.5, q_num=1, q_den=2)
    _run_trace(w, w.steps, with_pool=False)


def test_rebuild_grow_and_keep_all():
    import torch
    import moe_expert_layer_02_amd as m
    w = C.Workload(cid=96, name="grow", hidden=256, inter=128, n_experts=16, top_k=2, route=0,
                   n_layers=2, n_slots=6, t_decode=2, steps=10, zipf_alpha=1.0, keep_prob=0.5)
    runner, _ = _run_trace(w, w.steps, with_pool=False)
    sim_owner = runner.cache.owner.cpu().numpy()
    new = m.DeviceCache(9, w.n_layers, w.n_experts, runner.S, with_data=True)
    old = m.DeviceCache(6, w.n_layers, w.n_experts, runner.S, with_data=True)
    old.table.copy_(runner.cache.table)
    old.owner.copy_(runner.cache.owner)
    old.ts.copy_(runner.cache.ts)
    old.data.copy_(torch.arange(old.data.numel(), device="cuda", dtype=torch.int64).to(torch.uint8))
    m.cache_rebuild(old, new)
    torch.cuda.synchronize()
    sim = ocache.CacheSim(6, w.n_layers, w.n_experts)
    sim.table[:] = old.table.cpu().numpy()
    sim.owner[:] = old.owner.cpu().numpy()
    sim.ts[:] = old.ts.cpu().numpy()
    ref = sim.rebuild(9)
    assert np.array_equal(new.table.cpu().numpy(), ref.table)
    assert np.array_equal(new.owner.cpu().numpy(), ref.owner)
    assert np.array_equal(new.ts.cpu().numpy(), ref.ts)
    S = runner.S
    for old_s, new_s in sim.moves_of_rebuild(9):
        assert torch.equal(new.data[new_s * S:(new_s + 1) * S], old.data[old_s * S:(old_s + 1) * S])
    assert (sim_owner >= 0).sum() == (new.owner.cpu().numpy() >= 0).sum()
