"""Benchmark of one MoE layer's forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload qwen_decode|...]

Prints one JSON line.  The default workload is the Qwen-35B-A3B-like decode
stream: 40 stacked MoE layers per step, one token per step, softmax top-8,
int4 affine group-64 experts (1.77 MB each) in an 18.1 GB pool behind a
2048-slot HBM expert cache with LRU eviction.  A step is one pass of the whole
hot path over every layer: route -> classify_evict (dedup, hit/miss, K-victim
LRU, slot update) -> cache_fill -> decode expert FFN with the combine.  The
metric is expert-weight bytes streamed per second (|U| * S per layer call).

Other workloads (not the default line): ``ds_decode`` (DeepSeek-like sigmoid
group routing, MXFP4, batch 16) and ``qwen_prefill`` / ``ds_prefill``.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# sources of the decode FFN kernels (a recorded traffic figure is void once they change)
DECODE_SOURCES = ["moe_expert_layer_02_amd/csrc/decode.hip", "moe_expert_layer_02_amd/csrc/internal.h",
                  "moe_expert_layer_02_amd/csrc/classify_dev.h", "moe_expert_layer_02_amd/csrc/route_dev.h"]
PREFILL_SOURCES = ["moe_expert_layer_02_amd/csrc/prefill.hip", "moe_expert_layer_02_amd/csrc/internal.h"]
METRIC = "decode MoE-layer expert-weight GB/s (% HBM peak); prefill tokens/s (% MFMA peak)"


def _x_dev(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def cpu_baseline_decode(w, trace, n_calls: int, budget_s: float):
    """The oracle (fp32, NumPy BLAS) on a bounded sample of the same decode calls."""
    from oracle import ffn as offn
    from oracle import route as oroute
    from workloads import configs as C
    from workloads import experts as wx
    from workloads import traces as tr
    S = wx.expert_bytes(w.wfmt, w.hidden, w.inter)
    calls = [(s, l) for s in range(trace.steps) for l in range(w.n_layers)][:n_calls]
    nbytes = 0
    done = 0
    dt = 0.0
    for s, l in calls:
        # inputs of one call (not timed), generated call by call: a DS-like call's
        # experts alone are about 0.75 GB
        ids, wt = oroute.route(trace.logits[s, l], w.top_k, w.route, w.n_group, w.topk_group,
                               w.route_scale)
        blobs = {int(e): wx.expert_blob(C.seed(w.cid, 0), l * w.n_experts + int(e), w.wfmt,
                                        w.hidden, w.inter) for e in np.unique(ids)}
        x = tr.x_as_f32(tr.decode_x(w, s, l))
        t0 = time.perf_counter()
        offn.moe_layer(x, ids, wt, blobs.__getitem__, w.wfmt, w.hidden, w.inter, dtype=np.float32)
        dt += time.perf_counter() - t0
        nbytes += len(blobs) * S
        done += 1
        if dt > budget_s:
            break
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        cores = os.cpu_count() or 1
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{done} layer calls (first calls of the trace), fp32 NumPy dequant + "
                      f"GEMV + combine, {dt:.1f} s"}


def bench_decode(args, w, pool=None, q=None, roofline=True):
    """Timed region: K decode steps, each one replay of a captured graph holding
    the step's 40 (or 24) layer calls, after the step's inputs (logits,
    activations, tick base) are staged in HBM.  Layer call order "fused":
    decode_layer (route + classify/evict in one kernel, then the expert FFN with
    fill-through and the combine).  Order "split": route_plan and the FFN on the
    main stream, evict_fill (LRU update + fill copy) on a second stream that the
    next layer's route_plan waits for.

    Roofline: the expert FFN kernel timed with HIP events in a second, eager
    pass over the same trace (route, classify_evict, cache_fill as separate
    calls, then the FFN between two events on the same stream)."""
    import torch
    import moe_expert_layer_02_amd as m
    from workloads import experts as wx
    from workloads import gpu as wg
    from workloads import traces as tr

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    desc = m.LayerDesc(w.hidden, w.inter, w.n_experts, w.top_k, w.route, w.n_group,
                       w.topk_group, w.route_scale, w.wfmt)
    S = wx.expert_bytes(w.wfmt, w.hidden, w.inter)
    L, T = w.n_layers, w.t_decode
    n_trace = w.steps
    trace = tr.DecodeTrace(w, n_trace)
    if pool is None:
        pool = wg.make_pool(w, pack=lambda src, dst, n: m.pack_experts(desc, src, dst, n))
    K = w.victims_k
    policy = m.EvictPolicy(K, *(q if q is not None else (w.q_num, w.q_den)))
    cap = max(K, min(T * w.top_k, w.n_experts))
    logits_all = torch.from_numpy(trace.logits).to(dev)                      # [steps, L, T, E]
    xs_all = torch.stack([torch.stack([_x_dev(tr.decode_x(w, s, l), torch) for l in range(L)])
                          for s in range(n_trace)])                           # [steps, L, T, H]
    order = args.order if args.order != "auto" else "fused"

    class Step:
        def __init__(self):
            self.cache = m.DeviceCache(w.n_slots, L, w.n_experts, S)
            self.logits = torch.empty_like(logits_all[0])
            self.x = torch.empty_like(xs_all[0])
            self.tick = torch.zeros(1, dtype=torch.int64, device=dev)
            self.ids = torch.empty((L, T, w.top_k), dtype=torch.int32, device=dev)
            self.wt = torch.empty((L, T, w.top_k), dtype=torch.float32, device=dev)
            self.lists = [m.DeviceClassifyOut(cap) for _ in range(L)]
            self.out = torch.empty((L, T, w.hidden), dtype=torch.float32, device=dev)
            self.ws = torch.zeros(m.workspace_bytes(desc, T, m.MODE_DECODE), dtype=torch.uint8,
                                  device=dev)
            self.side = torch.cuda.Stream()
            self.planned = [torch.cuda.Event() for _ in range(L)]

        def stage(self, s):
            self.logits.copy_(logits_all[s % n_trace])
            self.x.copy_(xs_all[s % n_trace])
            self.tick.fill_(s * L)

        def layers(self):
            main = torch.cuda.current_stream()
            if order == "fused":
                for l in range(L):
                    m.decode_layer(desc, self.cache, pool, l, self.tick, l + 1, self.logits[l],
                                   self.x[l], policy, self.ids[l], self.wt[l], self.lists[l],
                                   self.out[l], self.ws)
                return
            self.side.wait_stream(main)
            for l in range(L):
                main.wait_stream(self.side)          # previous layer's slot update and fill
                m.route_plan(desc, self.cache, l, self.logits[l], self.ids[l], self.wt[l],
                             self.lists[l])
                self.planned[l].record(main)
                m.expert_ffn_decode(desc, self.x[l], self.ids[l], self.wt[l], self.cache, pool, l,
                                    self.lists[l], self.out[l], self.ws)
                self.side.wait_event(self.planned[l])
                m.evict_fill(desc, self.cache, pool, l, self.tick, l + 1, self.ids[l], policy,
                             self.lists[l], stream=self.side)
            main.wait_stream(self.side)

    warm = Step()                       # first launches (occupancy queries) outside capture
    warm.stage(0)
    warm.layers()
    torch.cuda.synchronize()
    del warm
    st = Step()
    st.stage(0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.layers()
    torch.cuda.synchronize()

    for s in range(args.warmup):
        st.stage(s)
        graph.replay()
    torch.cuda.synchronize()
    uniq_per_step = []
    stream = torch.cuda.current_stream()
    step_ev = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        st.stage(args.warmup + i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        step_ev.append((e0, e1))
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    m.check_error(st.ws, what="timed decode steps")   # no bounded wait gave up, no range flag
    replay_s = sum(a.elapsed_time(b) for a, b in step_ev) / 1e3   # the layer calls alone
    # distinct experts per call, from the trace's target sets (the routed top-k sets;
    # checked below against the device counts of the last step)
    for i in range(args.steps):
        s = (args.warmup + i) % n_trace
        for l in range(L):
            uniq_per_step.append(len(np.unique(trace.targets[s, l])))
    n_uniq = int(np.sum(uniq_per_step))
    last = (args.warmup + args.steps - 1) % n_trace
    for l in range(L):
        assert int(st.lists[l].counts[0].item()) == len(np.unique(trace.targets[last, l]))
    bytes_total = n_uniq * S
    n_calls = args.steps * L
    value = bytes_total / dt / 1e9
    if not roofline:
        return {"value": round(value, 2), "unit": "GB/s", "ms_per_step": round(dt / args.steps * 1e3, 4),
                "replay_ms_per_step": round(replay_s / args.steps * 1e3, 4), "steps": args.steps,
                "policy_q": [policy.q_num, policy.q_den]}

    # roofline pass: the FFN kernels alone.  Each step's bookkeeping (route,
    # classify_evict, cache_fill) runs eagerly for all layers first; then the
    # step's L FFN calls, one per layer (each reading its own layer's experts, as
    # in the real step), are captured into a graph whose replay is bracketed by
    # two events on the replay stream.  There are no host gaps inside the
    # bracket, so the per-launch time is the kernels' own (plus the graph's
    # inter-kernel gaps).
    rp = Step()
    rp_steps = min(args.steps, 10)
    u_rp = 0
    ev = []
    for s in range(args.warmup + rp_steps):
        rp.stage(s)
        for l in range(L):
            m.route(desc, rp.logits[l], rp.ids[l], rp.wt[l])
            m.classify_evict(rp.cache, l, s * L + l + 1, rp.ids[l], policy, rp.lists[l])
            m.cache_fill(rp.cache, pool, l, rp.lists[l], K)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for l in range(L):
                m.expert_ffn_decode(desc, rp.x[l], rp.ids[l], rp.wt[l], rp.cache, pool, l,
                                    rp.lists[l], rp.out[l], rp.ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        if s >= args.warmup:
            ev.append(e0.elapsed_time(e1) / L)
            u_rp += sum(len(np.unique(trace.targets[s % n_trace, l])) for l in range(L))
        del g
    m.check_error(rp.ws, what="roofline FFN calls")
    ffn_avg_s = float(np.mean(ev)) / 1e3
    n_launch = len(ev) * L
    per_call_bytes = u_rp * S / n_launch
    achieved = per_call_bytes / ffn_avg_s / 1e9
    ffn_roof = {"bound": "hbm", "kernel": ffn_kernel_label(w, T),
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_record(f"decode_ffn_{w.name}_traffic.md", DECODE_SOURCES),
                "bytes_per_launch": round(per_call_bytes),
                "avg_launch_us": round(ffn_avg_s * 1e6, 2), "launches_timed": n_launch}
    if small_call(w, T) and order == "fused":
        # the timed step is one layer_small_kernel launch per layer call: that is
        # the dominant kernel, priced on the expert bytes it must stream
        layer_s = replay_s / n_calls
        layer_bytes = bytes_total / n_calls
        roof = {"bound": "hbm",
                "kernel": "decode_layer: layer_small_kernel (bookkeeping and expert FFN, one launch "
                          "per layer call; event-timed over the timed steps' graph replays)",
                "achieved": round(layer_bytes / layer_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(layer_bytes / layer_s / 1e9 / HBM_PEAK_GBS, 4),
                "traffic": traffic_record(f"decode_layer_{w.name}_traffic.md", DECODE_SOURCES),
                "bytes_per_launch": round(layer_bytes), "avg_launch_us": round(layer_s * 1e6, 2),
                "launches_timed": n_calls, "ffn_call": ffn_roof}
    else:
        roof = ffn_roof
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(dt / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16" if w.wfmt == 0 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": L, "tokens_per_step": T, "hidden": w.hidden,
                   "inter": w.inter, "experts": w.n_experts, "top_k": w.top_k,
                   "weights": "int4_g64" if w.wfmt == 0 else "mxfp4", "cache_slots": w.n_slots,
                   "expert_bytes": S, "layer_calls_timed": n_calls, "parallelism": "single_gpu",
                   "order": order, "step": "one replay of a captured graph of the step's layer calls"},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decode(w, trace, n_calls=args.cpu_calls,
                                                  budget_s=args.cpu_budget)
    return res


def small_call(w, T):
    """The library's small-call rule: one launch for the expert FFN, and (with a
    cache of at most 2048 slots and 256 experts) one launch for a whole layer call."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    u = min(T * w.top_k, w.n_experts)
    return (T <= 16 and w.hidden in (1024, 2048, 4096) and u * (w.inter // 16) <= cus
            and u * (w.inter // 128) <= 32 and T * w.top_k * w.inter * 4 <= 32768
            and w.n_slots <= 2048 and w.n_experts <= 256 and T * w.top_k <= 128
            and w.victims_k <= 128)


def ffn_kernel_label(w, T):
    """Which kernels one expert_ffn_decode call launches for this workload."""
    if small_call(w, T):
        return ("expert_ffn_decode: ffn_small_kernel (one launch; inside a decode step the "
                "same work runs in layer_small_kernel together with the bookkeeping)")
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    u = min(T * w.top_k, w.n_experts)
    # the library's rule for the down pass with h in LDS (many distinct experts)
    if (u * (w.hidden // 32) >= 2 * cus * 8 and w.hidden % 512 == 0
            and 16 * (w.inter // 4 + 1) * 16 <= 135168):
        return "expert_ffn_decode: gate_up_kernel + down_lds_kernel (one call, two launches)"
    return "expert_ffn_decode: gate_up_kernel + down_kernel (one call, two launches)"


MFMA_PEAK_BF16_TFLOPS = 2500.0
# dense fp8 matrix-core peak: the rate of the scaled f8f6f4 MFMA when one operand is FP8
MFMA_PEAK_FP8_TFLOPS = 5000.0


def cpu_baseline_prefill(w, x_bits, ids, wt, budget_s: float, n_tok: int = 0, mx: bool = False):
    """The oracle (fp32, NumPy BLAS) on the prefill layer: every token when
    n_tok is 0, else the first n_tok tokens.  mx: the MX-activation layer
    (float64, as the oracle defines it)."""
    from oracle import ffn as offn
    from workloads import configs as C
    from workloads import experts as wx
    from workloads import traces as tr
    n_tok = n_tok or w.t_prefill
    toks = np.arange(n_tok)
    blobs = {int(e): wx.expert_blob(C.seed(w.cid, 0), int(e), w.wfmt, w.hidden, w.inter)
             for e in np.unique(ids[toks])}
    x = tr.x_as_f32(x_bits[toks])
    t0 = time.perf_counter()
    if mx:
        offn.moe_layer_mx8(x, ids[toks], wt[toks], blobs.__getitem__, w.hidden, w.inter)
    else:
        offn.moe_layer(x, ids[toks], wt[toks], blobs.__getitem__, w.wfmt, w.hidden, w.inter,
                       dtype=np.float32)
    dt = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        cores = os.cpu_count() or 1
    return {"value": round(n_tok / dt, 2), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": (f"the whole layer ({n_tok} tokens)" if n_tok == w.t_prefill else
                       f"first {n_tok} of {w.t_prefill} tokens") +
                      f", fp32 NumPy dequant of {len(blobs)} experts + GEMMs + combine, {dt:.1f} s"}


def bench_prefill(args, w, mx=False):
    import torch
    import moe_expert_layer_02_amd as m
    from workloads import experts as wx
    from workloads import gpu as wg
    from workloads import traces as tr

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    desc = m.LayerDesc(w.hidden, w.inter, w.n_experts, w.top_k, w.route, w.n_group,
                       w.topk_group, w.route_scale, w.wfmt)
    S = wx.expert_bytes(w.wfmt, w.hidden, w.inter)
    T, k = w.t_prefill, w.top_k
    x_bits = tr.prefill_x(w)
    logits_np = tr.prefill_logits(w)
    layer = wg.make_experts(w, 0, w.n_experts, C_seed(w),
                            pack=lambda src, dst, n: m.pack_experts(desc, src, dst, n))
    x = _x_dev(x_bits, torch)
    logits = torch.from_numpy(logits_np).to(dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    wt = torch.empty((T, k), dtype=torch.float32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    offsets = torch.empty(w.n_experts + 1, dtype=torch.int32, device=dev)
    wsp = torch.empty(m.workspace_bytes(desc, T, m.MODE_PERMUTE), dtype=torch.uint8, device=dev)
    ws = torch.empty(m.workspace_bytes(desc, T, m.MODE_PREFILL_MX if mx else m.MODE_PREFILL),
                     dtype=torch.uint8, device=dev)
    ffn = m.expert_ffn_prefill_mx if mx else m.expert_ffn_prefill
    out = torch.empty((T, w.hidden), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(events=None):
        m.route(desc, logits, ids, wt)
        m.permute(desc, ids, perm, offsets, wsp)
        if events is not None:
            events[0].record(stream)
        ffn(desc, x, ids, wt, layer, perm, offsets, out, ws)
        if events is not None:
            events[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    m.check_error(ws, m.MODE_PREFILL, what="timed prefill calls")
    ffn_s = float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3
    flops = 6.0 * w.hidden * w.inter * T * k          # algorithmic: gate, up, down
    achieved = flops / ffn_s / 1e12
    peak = MFMA_PEAK_FP8_TFLOPS if mx else MFMA_PEAK_BF16_TFLOPS
    res = {
        "metric": METRIC, "value": round(T * args.steps / dt, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(dt / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3 x fp4e2m1 (MX)" if mx else ("f16" if w.wfmt == 0 else "bf16"),
        "data": "synthetic",
        "config": {"workload": w.name + ("_mx_activations" if mx else ""), "tokens": T,
                   "hidden": w.hidden, "inter": w.inter,
                   "experts": w.n_experts, "top_k": k,
                   "weights": "int4_g64" if w.wfmt == 0 else "mxfp4",
                   "parallelism": "single_gpu"},
        "roofline": {"bound": "mfma",
                     "kernel": "expert_ffn_prefill_mx (plan_kernel + mx8_x_kernel + gate_up_mx + "
                               "down_mx + combine_rows_kernel)" if mx
                     else ("expert_ffn_prefill (plan_kernel + " + ("x16_kernel + " if w.wfmt == 0 else "") +
                           "gate_up_mfma + down_mfma + combine_rows_kernel)"),
                     "achieved": round(achieved, 1), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic_record(f"prefill_ffn_{w.name}{'_mx' if mx else ''}_traffic.md",
                                              PREFILL_SOURCES),
                     "flops_per_launch": flops,
                     "avg_launch_us": round(ffn_s * 1e6, 1)},
    }
    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        # the whole Qwen-like layer finishes in seconds on the host; the DS-like one
        # takes minutes, so it is timed on its first 512 tokens
        n_tok = 0 if w.t_prefill * w.hidden * w.inter <= 8192 * 2048 * 512 else 512
        if mx:
            n_tok = 128
        res["cpu_baseline"] = cpu_baseline_prefill(w, x_bits, ids.cpu().numpy(), wt.cpu().numpy(),
                                                   args.cpu_budget, n_tok, mx=mx)
    return res


def bench_miss_replay(args):
    """Decode expert miss rate versus cache size (percent of the expert pool) for
    the global LRU (the library's routing and bookkeeping calls on the GPU)
    against static hot-expert pinning and static whole-layer placement, replayed
    on identical synthetic routing traces (one token per step)."""
    import torch
    from moe_expert_layer_02_amd import replay
    from workloads import configs as C
    from workloads import traces as tr
    fracs = (0.05, 0.11, 0.2, 0.37, 0.5, 0.75)
    curves = {}
    t0 = time.perf_counter()
    for w in (C.QWEN_DECODE, C.DS_DECODE_SINGLE):
        import moe_expert_layer_02_amd as m
        desc = m.LayerDesc(w.hidden, w.inter, w.n_experts, w.top_k, w.route, w.n_group,
                           w.topk_group, w.route_scale, w.wfmt)
        trace = tr.DecodeTrace(w, w.steps)
        L, E = w.n_layers, w.n_experts
        rows = []
        for f in fracs:
            N = int(round(f * L * E))
            K = min(w.t_decode * w.top_k, E, N)
            lru, routed = replay.lru_misses(desc, trace.logits, N, K)
            rows.append({"cache_frac": f, "slots": N,
                         "lru": round(replay.miss_rate(lru), 4),
                         # the second half of the trace: no cold-start first touches
                         "lru_steady": round(replay.miss_rate(lru[w.steps // 2:]), 4),
                         "hot_pinned": round(replay.miss_rate(replay.hot_pinned_misses(routed, E, N)), 4),
                         "layer_static": round(replay.miss_rate(replay.layer_static_misses(routed, E, N)), 4)})
            print(f"miss replay {w.name} {f:.0%}: {rows[-1]}", file=sys.stderr, flush=True)
        curves[w.name] = {"layers": L, "experts": E, "top_k": w.top_k, "steps": w.steps,
                          "calls": w.steps * L, "points": rows}
        torch.cuda.synchronize()
    return {"metric": "decode expert-cache miss rate vs cache size (fraction of the expert pool)",
            "unit": "misses / distinct routed experts", "n_gpus": 1, "data": "synthetic",
            "higher_is_better": False, "policies": {
                "lru": "global LRU across layers (library routing + classify_evict on the GPU)",
                "lru_steady": "the same LRU run, misses counted over the second half of the trace",
                "hot_pinned": "the N most frequently routed (layer, expert) pairs of the replayed "
                              "trace itself, fixed (a clairvoyant static placement)",
                "layer_static": "whole layers 0.. resident while they fit, fixed"},
            "curves": curves, "wall_s": round(time.perf_counter() - t0, 1)}


def bench_prefill_pipeline(args, w, n_layers: int):
    """Prefill of n_layers consecutive layers with the experts streamed from a
    pinned host pool (moe355_prefill_layers): two whole-layer buffers (the
    copy of layer l+1 overlaps layer l), one buffer (copies and compute in
    series), the compute alone from a resident buffer, and the copies alone
    (the pinned host-to-device bandwidth B_P).  Every timed region starts with
    both streams idle and ends when both are done."""
    import torch
    import moe_expert_layer_02_amd as m
    from workloads import experts as wx
    from workloads import gpu as wg
    from workloads import traces as tr
    desc = m.LayerDesc(w.hidden, w.inter, w.n_experts, w.top_k, w.route, w.n_group,
                       w.topk_group, w.route_scale, w.wfmt)
    T, E, k = w.t_prefill, w.n_experts, w.top_k
    S = wx.expert_bytes(w.wfmt, w.hidden, w.inter)
    LB = E * S
    pool_dev = wg.make_pool(w, n_layers=n_layers,
                            pack=lambda src, dst, n: m.pack_experts(desc, src, dst, n))
    host_pool = torch.empty(pool_dev.numel(), dtype=torch.uint8, pin_memory=True)
    host_pool.copy_(pool_dev)
    del pool_dev
    logits = [torch.from_numpy(tr.prefill_logits_layer(w, l)).cuda() for l in range(n_layers)]
    xs = [torch.from_numpy(tr.prefill_x_layer(w, l).view(np.int16)).cuda().view(torch.bfloat16)
          for l in range(n_layers)]
    outs = [torch.empty((T, w.hidden), dtype=torch.float32, device="cuda") for _ in range(n_layers)]
    bufs = [torch.empty(LB, dtype=torch.uint8, device="cuda") for _ in range(2)]
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, k), dtype=torch.float32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    ws = torch.empty(m.workspace_bytes(desc, T, m.MODE_PREFILL), dtype=torch.uint8, device="cuda")
    wsp = torch.empty(m.workspace_bytes(desc, T, m.MODE_PERMUTE), dtype=torch.uint8, device="cuda")
    main, copy = torch.cuda.current_stream(), torch.cuda.Stream()

    def timed(fn, reps):
        ts = []
        for _ in range(reps):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(main)
            copy.wait_stream(main)
            fn()
            main.wait_stream(copy)
            e1.record(main)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        return float(np.median(ts))

    def pipeline(double):
        return lambda: m.prefill_layers(desc, host_pool, bufs, logits, xs, outs, ids, wt, perm,
                                        offsets, ws, wsp, double, copy_stream=copy)

    def resident():
        for l in range(n_layers):
            m.route(desc, logits[l], ids, wt)
            m.permute(desc, ids, perm, offsets, wsp)
            m.expert_ffn_prefill(desc, xs[l], ids, wt, bufs[0], perm, offsets, outs[l], ws)

    def copies():
        with torch.cuda.stream(copy):
            for l in range(n_layers):
                bufs[l % 2].copy_(host_pool[l * LB:(l + 1) * LB], non_blocking=True)

    reps = max(1, min(args.steps, 5))
    pipeline(True)()          # warm-up: first launches, LDS attributes
    torch.cuda.synchronize()
    t2, t1 = timed(pipeline(True), reps), timed(pipeline(False), reps)
    tc, tcopy = timed(resident, reps), timed(copies, reps)
    m.check_error(ws, m.MODE_PREFILL, what="pipelined prefill")
    tok = T * n_layers
    return {"metric": "prefill tokens/s with the experts streamed from pinned host memory",
            "value": round(tok / t2, 1), "unit": "tokens/s", "n_gpus": 1, "steps": reps,
            "higher_is_better": True, "data": "synthetic",
            "dtype": "f16" if w.wfmt == 0 else "bf16",
            "config": {"workload": w.name + "_pipelined", "layers": n_layers, "tokens": T,
                       "layer_bytes": LB, "parallelism": "single_gpu"},
            "two_buffers_s": round(t2, 5), "one_buffer_s": round(t1, 5),
            "compute_only_s": round(tc, 5), "copies_only_s": round(tcopy, 5),
            "B_P_GBs": round(LB * n_layers / tcopy / 1e9, 2),
            "one_buffer_tokens_per_s": round(tok / t1, 1),
            "loss_without_second_buffer": round(1.0 - t2 / t1, 4),
            "overlap_of_compute": round((tc + tcopy - t2) / tc, 4)}


def bench_decode_host_pool(args):
    """The Qwen-like decode stream with the expert pool in pinned host memory
    (the host tier): B_P is the pinned host-to-device DMA rate of one layer of
    experts; B_H the rate at which the decode FFN computes experts in place
    straight from that pool (every expert of a step's calls read over PCIe);
    q* = m * B_P / B_H (rounded, clamped to m).  The step is then timed under
    that split, under pure fill (q = m) and under no fill (q = 0: every miss
    computed in place from host memory, the cache never filled)."""
    import torch
    from fractions import Fraction
    import moe_expert_layer_02_amd as m
    from workloads import configs as C
    from workloads import experts as wx
    from workloads import gpu as wg
    from workloads import traces as tr
    w = C.QWEN_DECODE
    desc = m.LayerDesc(w.hidden, w.inter, w.n_experts, w.top_k, w.route, w.n_group,
                       w.topk_group, w.route_scale, w.wfmt)
    S, E, L = wx.expert_bytes(w.wfmt, w.hidden, w.inter), w.n_experts, w.n_layers
    t0 = time.perf_counter()
    pool_dev = wg.make_pool(w, pack=lambda src, dst, n: m.pack_experts(desc, src, dst, n))
    host = torch.empty(pool_dev.numel(), dtype=torch.uint8, pin_memory=True)
    host.copy_(pool_dev)
    del pool_dev
    torch.cuda.empty_cache()
    setup_s = time.perf_counter() - t0
    stream = torch.cuda.current_stream()

    def med_time(fn, reps=5):
        ts = []
        for _ in range(reps):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        return float(np.median(ts))

    # B_P: one layer of experts (E * S bytes) by DMA
    buf = torch.empty(E * S, dtype=torch.uint8, device="cuda")
    t_copy = med_time(lambda: buf.copy_(host[:E * S], non_blocking=True))
    B_P = E * S / t_copy / 1e9
    del buf
    # B_H: one step's 40 FFN calls with every routed expert read in place from the host pool
    trace = tr.DecodeTrace(w, 2)
    T = w.t_decode
    ids = torch.empty((L, T, w.top_k), dtype=torch.int32, device="cuda")
    wt = torch.empty((L, T, w.top_k), dtype=torch.float32, device="cuda")
    lg = torch.from_numpy(trace.logits[0]).cuda()
    xs = torch.stack([_x_dev(tr.decode_x(w, 0, l), torch) for l in range(L)])
    outs = torch.empty((L, T, w.hidden), dtype=torch.float32, device="cuda")
    lists = [m.DeviceClassifyOut(min(T * w.top_k, E)) for _ in range(L)]
    ws = torch.zeros(m.workspace_bytes(desc, T, m.MODE_DECODE), dtype=torch.uint8, device="cuda")
    for l in range(L):
        m.route(desc, lg[l], ids[l], wt[l])
        m.dedup(ids[l], E, lists[l])

    def in_place_step():
        for l in range(L):
            m.expert_ffn_decode(desc, xs[l], ids[l], wt[l], None, host, l, lists[l], outs[l], ws)
    in_place_step()
    t_inplace = med_time(in_place_step)
    m.check_error(ws, what="in-place FFN calls from host memory")
    n_uniq = sum(int(lists[l].counts[0].item()) for l in range(L))
    B_H = n_uniq * S / t_inplace / 1e9
    ratio = Fraction(B_P / B_H).limit_denominator(64)
    q_star = (ratio.numerator, ratio.denominator)
    policies = {"q_star": q_star, "pure_fill": (1, 1), "no_fill": (0, 1)}
    res = {"metric": "decode MoE-layer steps with the expert pool in pinned host memory",
           "unit": "ms per step", "n_gpus": 1, "higher_is_better": False, "data": "synthetic",
           "config": {"workload": w.name + "_host_pool", "layers": L, "tokens_per_step": T,
                      "pool_bytes": int(host.numel()), "cache_slots": w.n_slots},
           "B_P_GBs": round(B_P, 2), "B_H_GBs": round(B_H, 2),
           "q_star": f"q = round(m * {q_star[0]} / {q_star[1]}), clamped to m",
           "setup_s": round(setup_s, 1), "policies": {}}
    for name, q in policies.items():
        r = bench_decode(args, w, pool=host, q=q, roofline=False)
        res["policies"][name] = r
        print(f"host pool {name}: {r}", file=sys.stderr, flush=True)
    return res


def bench_decode_floor(args):
    """What a decode step's 40 graph nodes cost before any expert work: graphs
    of 40 dependent nodes on one stream, each replay preceded by a 1 GiB read
    that evicts the lines the nodes touch (L2 and the memory-side cache), then
    timed with HIP events around the replay alone.  Nodes: an empty-work kernel
    of one workgroup (a one-element add), a 1 MiB fill (hundreds of
    workgroups), one dependent cold read (a one-element copy from a separate
    cold 2 MiB page per node: launch + one HBM round trip + the store), and a
    7 MiB copy per node from 40 distinct sources (14 MiB moved, the size of a
    Qwen-like layer call's expert bytes)."""
    import torch
    dev = torch.device("cuda:0")
    L, reps = 40, max(5, args.steps)
    page = 1 << 21
    one = torch.zeros(1, dtype=torch.float32, device=dev)
    fill = torch.empty(513 * 512, dtype=torch.float32, device=dev)
    src = torch.zeros(L * page // 4, dtype=torch.float32, device=dev)
    dst = torch.zeros(L, dtype=torch.float32, device=dev)
    n7 = (7 << 20) // 2
    big = torch.zeros((L, n7), dtype=torch.bfloat16, device=dev)
    out7 = torch.empty(n7, dtype=torch.bfloat16, device=dev)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)      # 1 GiB
    nodes = {
        "empty_node": lambda l: one.add_(1.0),
        "fill_1MiB_node": lambda l: fill.fill_(float(l)),
        "cold_read_node": lambda l: dst[l:l + 1].copy_(src[l * (page // 4):l * (page // 4) + 1]),
        "copy_7MiB_node": lambda l: out7.copy_(big[l]),
    }
    stream = torch.cuda.current_stream()
    res = {"metric": "decode graph-node floor", "unit": "us per node", "n_gpus": 1,
           "nodes_per_graph": L, "replays": reps, "data": "synthetic",
           "config": {"workload": "decode_floor", "parallelism": "single_gpu"}}
    for name, fn in nodes.items():
        for l in range(L):
            fn(l)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for l in range(L):
                fn(l)
        torch.cuda.synchronize()
        ts = []
        for i in range(reps + 2):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            if i >= 2:
                ts.append(e0.elapsed_time(e1) * 1e3 / L)
        res[name] = round(float(np.median(ts)), 3)
        del g
    res["copy_7MiB_GBs"] = round(2 * n7 * 2 / (res["copy_7MiB_node"] * 1e-6) / 1e9, 1)
    return res


def C_seed(w):
    from workloads import configs as C
    return C.seed(w.cid, 0)


def calib_copy(mib: int, reps: int):
    """A plain device copy of known size, for scaling the HBM byte counters.

    Under ``rocprofv3 --pmc FETCH_SIZE`` (or WRITE_SIZE) each copy dispatch should
    read (write) ``mib`` MiB; the ratio of that to the counter's reading is the
    factor applied to the FFN kernels' readings.
    """
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"calib_copy_bytes": n, "dispatches": reps}


def traffic_record(name: str, sources: list[str]):
    """HBM bytes per launch from a committed PMC summary, if it still describes
    the current kernel sources (sha256 of the listed files), else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "|", " ")):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if rec.get("source_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in rec:
        return None
    return float(rec["traffic_bytes_per_launch"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen_decode",
                    choices=["qwen_decode", "ds_decode", "qwen_prefill", "ds_prefill",
                             "ds_prefill_mx", "miss_replay", "qwen_prefill_pipeline",
                             "ds_prefill_pipeline", "qwen_decode_host_pool", "decode_floor"])
    ap.add_argument("--order", default="auto", choices=["auto", "fused", "split"],
                    help="decode layer call order (auto: fused)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sub", action="store_true",
                    help="print the selected workload alone (the default Qwen-like decode line "
                         "also carries Qwen-like prefill and DS-like decode sub-records)")
    ap.add_argument("--cpu-calls", type=int, default=160)
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path is "
              "single-GPU by design", file=sys.stderr)
        sys.exit(2)
    if args.calib_copy:
        print(json.dumps(calib_copy(args.calib_copy, 5)), flush=True)
        return
    import moe_expert_layer_02_amd as m
    m.check_build()         # the library under test was built from these sources
    from workloads import configs as C
    if args.workload == "miss_replay":
        print(json.dumps(bench_miss_replay(args)), flush=True)
        return
    if args.workload == "decode_floor":
        print(json.dumps(bench_decode_floor(args)), flush=True)
        return
    if args.workload == "qwen_decode_host_pool":
        print(json.dumps(bench_decode_host_pool(args)), flush=True)
        return
    if args.workload.endswith("_pipeline"):
        w, n = (C.QWEN_PREFILL, 8) if args.workload.startswith("qwen") else (C.DS_STRESS, 4)
        print(json.dumps(bench_prefill_pipeline(args, w, n)), flush=True)
        return
    w = {"qwen_decode": C.QWEN_DECODE, "ds_decode": C.DS_DECODE, "qwen_prefill": C.QWEN_PREFILL,
         "ds_prefill": C.DS_STRESS, "ds_prefill_mx": C.DS_STRESS}[args.workload]
    if "prefill" in args.workload:
        res = bench_prefill(args, w, mx=args.workload.endswith("_mx"))
    else:
        res = bench_decode(args, w)
    if args.workload == "qwen_decode" and not args.no_sub:
        # the same step definition, timing and roofline rules on two more workloads
        import torch
        res["sub_records"] = []
        for name, fn, sw in (("qwen_prefill", bench_prefill, C.QWEN_PREFILL),
                             ("ds_decode", bench_decode, C.DS_DECODE)):
            torch.cuda.empty_cache()
            print(f"bench: sub-record {name}", file=sys.stderr, flush=True)
            res["sub_records"].append(fn(args, sw))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
