"""The decode-layer calls on the GPU, in both orders the library offers:
"fused" (route + classify_evict in one kernel, then the expert FFN with
fill-through) and "split" (route + plan, the FFN reading misses from the pool,
and the LRU update + fill copy on a second stream that the next layer waits
for).  Every call of decode traces bit-exact against the oracle's simulator on
the integer outputs, sampled layer outputs against the oracle, every cache slot
holding its owner's pool bytes afterwards, and a whole decode step captured as
a graph and replayed, each replay checked against eager execution."""
import numpy as np
import pytest

from oracle import cache as ocache
from oracle import ffn as offn
from oracle import route as oroute
from workloads import configs as C
from workloads import experts as wx
from workloads import traces as tr

from gpu_common import BlobSource, check_close, desc_of, packer, say

pytestmark = pytest.mark.gpu


def _x_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


class LayerRunner:
    def __init__(self, w, n_slots, pool, mode="fused"):
        import torch
        import moe_expert_layer_02_amd as m
        self.m, self.torch, self.w, self.mode = m, torch, w, mode
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

    def stage(self, step, logits_np, xs):
        self.logits.copy_(self.torch.from_numpy(logits_np))
        self.x.copy_(xs)
        self.tick.fill_(step * self.w.n_layers)

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


@pytest.mark.parametrize("mode", ["fused", "split"])
@pytest.mark.parametrize("cid,steps,sample", [(2, 64, [(0, 3), (63, 39)]), (4, 24, [(5, 7)]),
                                              (5, 24, [(23, 0)]), (6, 40, [(0, 1), (39, 3)]),
                                              (7, 40, [(1, 0), (39, 2)]), (8, 40, [(0, 2), (39, 1)]),
                                              (9, 40, [(0, 0), (39, 3)])])
def test_decode_layer_trace(cid, steps, sample, mode):
    import torch
    from workloads import gpu as wg
    w = C.ALL[cid] if cid in C.ALL else EXTRA[cid]
    say(f"decode_layer trace {w.name} ({mode}): {steps} steps")
    trace = tr.DecodeTrace(w, steps)
    pool = wg.make_pool(w, pack=packer(desc_of(w)))
    run = LayerRunner(w, w.n_slots, pool, mode)
    sim = ocache.CacheSim(w.n_slots, w.n_layers, w.n_experts)
    src = BlobSource(w)
    for s in range(steps):
        xs = _xs(w, s)
        run.stage(s, trace.logits[s], xs)
        run.step()
        torch.cuda.synchronize()
        for l in range(w.n_layers):
            rid, rw = oroute.route(trace.logits[s, l], w.top_k, w.route, w.n_group, w.topk_group,
                                   w.route_scale)
            exp = sim.classify_evict(l, s * w.n_layers + l + 1, rid, run.K, w.q_num, w.q_den)
            got = run.lists[l].host()
            assert got["counts"] == exp["counts"], (s, l, got["counts"], exp["counts"])
            for key in ("uniq", "hit_expert", "hit_slot", "miss", "fill_expert", "fill_slot",
                        "inplace", "victims"):
                assert got[key] == exp[key], (s, l, key)
            assert np.array_equal(run.ids[l].cpu().numpy(), rid)
            if (s, l) in sample:
                toks = list(range(min(2, w.t_decode)))
                want = offn.moe_layer(tr.x_as_f32(tr.decode_x(w, s, l)), rid, rw,
                                      lambda e: src(l, e), w.wfmt, w.hidden, w.inter, tokens=toks)
                check_close(run.out[l].cpu().numpy()[toks], want, f"{w.name} call ({s},{l})")
    assert np.array_equal(run.cache.table.cpu().numpy(), sim.table)
    assert np.array_equal(run.cache.ts.cpu().numpy(), sim.ts)
    S = run.S
    owner = run.cache.owner.cpu().numpy()
    data, pv = run.cache.data.view(-1, S), pool.view(-1, S)
    occ = np.nonzero(owner >= 0)[0]
    for i in range(0, len(occ), 64):
        sl = torch.from_numpy(occ[i:i + 64]).cuda()
        ow = torch.from_numpy(owner[occ[i:i + 64]].astype(np.int64)).cuda()
        assert torch.equal(data.index_select(0, sl), pv.index_select(0, ow)), "slot bytes differ"
    say(f"{w.name}: {steps * w.n_layers} calls bit-exact, {len(occ)} slots hold their pool bytes")


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
    for s in range(6):
        for w, run, trace, src in runs:
            xs = _xs(w, s)
            run.stage(s, trace.logits[s], xs)
            run.step()
            torch.cuda.synchronize()
            assert int(ws_[:65536].count_nonzero()) == 0, (w.name, s)
            if s in (0, 5):
                l = s % w.n_layers
                rid, rw = oroute.route(trace.logits[s, l], w.top_k, w.route, w.n_group,
                                       w.topk_group, w.route_scale)
                want = offn.moe_layer(tr.x_as_f32(tr.decode_x(w, s, l)), rid, rw,
                                      lambda e: src(l, e), w.wfmt, w.hidden, w.inter)
                check_close(run.out[l].cpu().numpy(), want, f"{w.name} shared workspace ({s},{l})")
    say("workspace header zero after every step, two shapes sharing it")


@pytest.mark.parametrize("mode", ["fused", "split"])
def test_decode_step_graph_replay_matches_eager(mode):
    import torch
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
    eager = LayerRunner(w, w.n_slots, pool, mode)
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
    for s in range(steps):
        xs = _xs(w, s)
        eager.stage(s, trace.logits[s], xs)
        eager.step()
        torch.cuda.synchronize()
        graphed.stage(s, trace.logits[s], xs)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(eager.ids, graphed.ids), s
        # the combine adds a token's k contributions with atomics in no fixed order
        torch.testing.assert_close(graphed.out, eager.out, rtol=1e-6, atol=1e-5)
        assert torch.equal(eager.cache.table, graphed.cache.table), s
        assert torch.equal(eager.cache.ts, graphed.cache.ts), s
        say(f"graph replay {s} ({mode}) matches eager")
