"""Decode expert FFN parity on the GPU against the oracle: small shapes that
span several row tiles with ragged token counts, both weight formats, the
tiny whole-layer workload end to end, sampled calls of the full-size decode
workloads (experts read from cache slots and from the pool), and edge cases
(one expert shared by every token, the largest T*k, empty batch)."""
import numpy as np
import pytest

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


def _decode_whole_layer(w, x_bits, ids_np, wt_np, seed=None):
    """GPU decode FFN with every expert of one layer resident (no cache)."""
    import torch
    import moe_expert_layer_02_amd as m
    from workloads import gpu as wg
    seed = C.seed(w.cid, 0) if seed is None else seed
    S = wx.expert_bytes(w.wfmt, w.hidden, w.inter)
    desc = desc_of(w)
    layer = wg.make_experts(w, 0, w.n_experts, seed, pack=packer(desc))
    T = x_bits.shape[0]
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).cuda()
    wt = torch.from_numpy(np.ascontiguousarray(wt_np, dtype=np.float32)).cuda()
    exp = m.DeviceClassifyOut(max(1, min(T * w.top_k, w.n_experts)))
    m.dedup(ids, w.n_experts, exp)
    out = torch.full((T, w.hidden), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros(m.workspace_bytes(desc, T, m.MODE_DECODE), dtype=torch.uint8, device="cuda")
    m.expert_ffn_decode(desc, _x_dev(x_bits), ids, wt, None, layer, 0, exp, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _oracle_layer(w, x_bits, ids, wt, seed=None, tokens=None, layer=0):
    src = BlobSource(w, seed)
    return offn.moe_layer(tr.x_as_f32(x_bits), ids, wt, lambda e: src(layer, e), w.wfmt,
                          w.hidden, w.inter, tokens=tokens)


SMALL = [
    # (H, I, E, k, T, wfmt)
    (256, 128, 16, 2, 4, C.WFMT_INT4_G64),
    (512, 256, 32, 3, 5, C.WFMT_INT4_G64),
    (1024, 512, 24, 4, 7, C.WFMT_MXFP4),
    (2048, 512, 64, 8, 3, C.WFMT_INT4_G64),
    (2048, 1024, 40, 6, 9, C.WFMT_MXFP4),
    (4096, 2048, 16, 6, 2, C.WFMT_MXFP4),
    (4096, 256, 20, 5, 4, C.WFMT_INT4_G64),
    # few experts per call: eight-wavefront gate/up blocks and down split over I
    (1024, 512, 32, 4, 1, C.WFMT_INT4_G64),
    (4096, 1024, 16, 2, 1, C.WFMT_MXFP4),
    (1024, 256, 16, 2, 2, C.WFMT_INT4_G64),
]


def test_decode_small_call_sync_words_left_zero():
    """The one-launch small-call FFN (gate/up and down blocks counting through
    the workspace's first 65536 bytes) leaves those bytes zero after every call,
    the error word (byte 4608) included, and gives the same output on repeated
    calls: the down blocks sum the experts in a fixed order, and the two halves
    of each tile add onto zero in either order to the same value."""
    import torch
    import moe_expert_layer_02_amd as m
    from workloads import gpu as wg
    H, I, E, k, T = 2048, 512, 64, 8, 1
    w = C.Workload(cid=177, name="small-sync", hidden=H, inter=I, n_experts=E, top_k=k,
                   route=0, wfmt=C.WFMT_INT4_G64)
    say("decode small-call sync words")
    desc = desc_of(w)
    layer = wg.make_experts(w, 0, E, C.seed(w.cid, 0), pack=packer(desc))
    rng = np.random.default_rng(7)
    ws = torch.zeros(m.workspace_bytes(desc, T, m.MODE_DECODE), dtype=torch.uint8, device="cuda")
    outs = []
    for call in range(6):
        # three calls with fresh inputs, then the same inputs three times in a row
        r = rng if call < 3 else np.random.default_rng(11)
        x_bits = tr.bf16_normal(r, (T, H))
        ids_np, wt_np = oroute.softmax_topk(r.standard_normal((T, E)).astype(np.float32), k)
        ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).cuda()
        wt = torch.from_numpy(np.ascontiguousarray(wt_np, dtype=np.float32)).cuda()
        exp = m.DeviceClassifyOut(min(T * k, E))
        m.dedup(ids, E, exp)
        out = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
        m.expert_ffn_decode(desc, _x_dev(x_bits), ids, wt, None, layer, 0, exp, out, ws)
        torch.cuda.synchronize()
        assert int(ws[:65536].count_nonzero()) == 0, f"call {call}: sync words not cleared"
        outs.append(out.cpu().numpy())
        if call == 0:
            check_close(outs[0], _oracle_layer(w, x_bits, ids_np, wt_np), "small-call decode")
    assert np.array_equal(outs[3], outs[4]) and np.array_equal(outs[4], outs[5])


@pytest.mark.parametrize("H,I,E,k,T,wfmt", SMALL)
def test_decode_small_shapes(H, I, E, k, T, wfmt):
    w = C.Workload(cid=100 + H // 256 + I // 64 + E, name="small", hidden=H, inter=I,
                   n_experts=E, top_k=k, route=0, wfmt=wfmt)
    say(f"decode small H={H} I={I} E={E} k={k} T={T} fmt={wfmt}")
    rng = np.random.default_rng(H + I + E + k + T)
    x_bits = tr.bf16_normal(rng, (T, H))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, wt = oroute.softmax_topk(logits, k)
    got = _decode_whole_layer(w, x_bits, ids, wt)
    want = _oracle_layer(w, x_bits, ids, wt)
    check_close(got, want, f"decode H={H} I={I} fmt={wfmt}")


def test_decode_tiny_workload_end_to_end():
    """Tiny workload: x . W_r^T -> softmax top-2 -> dedup -> expert FFN, all on the GPU."""
    import torch
    import moe_expert_layer_02_amd as m
    w = C.TINY
    x_bits, wr = tr.tiny_inputs(w)
    lg = torch.empty((w.t_decode, w.n_experts), dtype=torch.float32, device="cuda")
    m.router_logits(desc_of(w), _x_dev(x_bits), torch.from_numpy(wr).cuda(), lg)
    ids = torch.empty((w.t_decode, w.top_k), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.t_decode, w.top_k), dtype=torch.float32, device="cuda")
    m.route(desc_of(w), lg, ids, wt)
    torch.cuda.synchronize()
    got = _decode_whole_layer(w, x_bits, ids.cpu().numpy(), wt.cpu().numpy())
    ref_logits = oroute.router_logits(tr.x_as_f32(x_bits), wr)
    rid, rw = oroute.softmax_topk(ref_logits, w.top_k)
    assert (ids.cpu().numpy() == rid).all()
    want = _oracle_layer(w, x_bits, rid, rw)
    check_close(got, want, "tiny workload")


def test_decode_one_expert_shared_by_all_tokens():
    w = C.Workload(cid=120, name="shared", hidden=2048, inter=512, n_experts=32, top_k=4,
                   route=0, wfmt=C.WFMT_INT4_G64)
    T = 13
    rng = np.random.default_rng(3)
    x_bits = tr.bf16_normal(rng, (T, w.hidden))
    ids = np.stack([np.r_[5, rng.choice([e for e in range(32) if e != 5], 3, replace=False)]
                    for _ in range(T)]).astype(np.int32)
    wt = rng.random((T, 4)).astype(np.float32)
    got = _decode_whole_layer(w, x_bits, ids, wt)
    check_close(got, _oracle_layer(w, x_bits, ids, wt), "one shared expert")


def test_decode_largest_pair_count():
    w = C.Workload(cid=121, name="maxpairs", hidden=1024, inter=256, n_experts=64, top_k=8,
                   route=0, wfmt=C.WFMT_MXFP4)
    T = 32   # T*k = 256, the decode limit
    rng = np.random.default_rng(4)
    x_bits = tr.bf16_normal(rng, (T, w.hidden))
    ids, wt = oroute.softmax_topk(rng.standard_normal((T, 64)).astype(np.float32), 8)
    got = _decode_whole_layer(w, x_bits, ids, wt)
    check_close(got, _oracle_layer(w, x_bits, ids, wt), "T*k=256")


@pytest.mark.parametrize("wfmt", [C.WFMT_MXFP4, C.WFMT_INT4_G64])
def test_decode_many_experts_window_restage(wfmt):
    """Many distinct experts (the h-in-LDS down pass): expert 0 takes all 32 tokens
    (two token groups of 16) and 224 other experts one pair each, so a block's
    items run past the 16-row h window and it restages; two tokens checked."""
    w = C.Workload(cid=122 + wfmt, name="window", hidden=4096, inter=2048, n_experts=256,
                   top_k=8, route=0, wfmt=wfmt)
    T = 32
    rng = np.random.default_rng(5 + wfmt)
    x_bits = tr.bf16_normal(rng, (T, w.hidden))
    others = rng.permutation(np.arange(1, 256))[:T * 7].reshape(T, 7)
    ids = np.concatenate([np.zeros((T, 1), dtype=np.int64), others], axis=1).astype(np.int32)
    wt = (0.05 + rng.random((T, 8))).astype(np.float32)
    got = _decode_whole_layer(w, x_bits, ids, wt)
    toks = [0, T - 1]
    want = _oracle_layer(w, x_bits, ids, wt, tokens=toks)
    check_close(got[toks], want, f"many experts, window restage (fmt {wfmt})")


def test_decode_many_experts_balanced_units():
    """The h-in-LDS down pass with 36 distinct experts (fewer 1024-row chunks
    than CUs): its 64-row units are dealt to the blocks in balanced ranges that
    cross expert boundaries, each block entering several token groups as
    phases.  Every token checked."""
    w = C.Workload(cid=126, name="units", hidden=4096, inter=2048, n_experts=256, top_k=6,
                   route=0, wfmt=C.WFMT_MXFP4)
    T = 6
    rng = np.random.default_rng(21)
    x_bits = tr.bf16_normal(rng, (T, w.hidden))
    ids = rng.permutation(256)[:T * 6].reshape(T, 6).astype(np.int32)   # 36 distinct experts
    wt = (0.05 + rng.random((T, 6))).astype(np.float32)
    got = _decode_whole_layer(w, x_bits, ids, wt)
    check_close(got, _oracle_layer(w, x_bits, ids, wt), "36 experts, balanced down units")


def test_decode_empty_batch_is_noop():
    import torch
    import moe_expert_layer_02_amd as m
    w = C.QWEN_DECODE
    desc = desc_of(w)
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    exp = m.DeviceClassifyOut(8)
    out = torch.empty((0, w.hidden), dtype=torch.float32, device="cuda")
    x = torch.empty((0, w.hidden), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    pool = torch.empty(16, dtype=torch.uint8, device="cuda")
    m.expert_ffn_decode(desc, x, e.view(0, 8), torch.empty((0, 8), device="cuda"), None, pool, 0,
                        exp, out, ws)
    torch.cuda.synchronize()


@pytest.mark.parametrize("cid,steps,sample", [(2, 6, [(0, 0), (2, 17), (5, 39)]),
                                              (4, 3, [(1, 5), (2, 23)])])
def test_decode_full_size_sampled_calls(cid, steps, sample):
    """Whole decode steps at full size through the cache; sampled calls checked."""
    import torch
    import moe_expert_layer_02_amd as m
    from workloads import gpu as wg
    w = C.ALL[cid]
    say(f"decode full size {w.name}: {steps} steps, sampled {sample}")
    desc = desc_of(w)
    trace = tr.DecodeTrace(w, steps)
    pool = wg.make_pool(w, pack=packer(desc_of(w)))
    S = wx.expert_bytes(w.wfmt, w.hidden, w.inter)
    cache = m.DeviceCache(w.n_slots, w.n_layers, w.n_experts, S)
    K = w.victims_k
    policy = m.EvictPolicy(K, w.q_num, w.q_den)
    exp = m.DeviceClassifyOut(max(K, min(w.t_decode * w.top_k, w.n_experts)))
    ids = torch.empty((w.t_decode, w.top_k), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.t_decode, w.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((w.t_decode, w.hidden), dtype=torch.float32, device="cuda")
    ws = torch.zeros(m.workspace_bytes(desc, w.t_decode, m.MODE_DECODE), dtype=torch.uint8,
                     device="cuda")
    src = BlobSource(w)
    rng = np.random.default_rng(cid)
    for s in range(steps):
        for l in range(w.n_layers):
            x_bits = tr.decode_x(w, s, l)
            lg = torch.from_numpy(trace.logits[s, l]).cuda()
            m.route(desc, lg, ids, wt)
            m.classify_evict(cache, l, s * w.n_layers + l + 1, ids, policy, exp)
            m.cache_fill(cache, pool, l, exp, K)
            m.expert_ffn_decode(desc, _x_dev(x_bits), ids, wt, cache, pool, l, exp, out, ws)
            if (s, l) in sample:
                torch.cuda.synchronize()
                h = exp.host()
                got = out.cpu().numpy()
                rid, rw = oroute.route(trace.logits[s, l], w.top_k, w.route, w.n_group,
                                       w.topk_group, w.route_scale)
                assert (ids.cpu().numpy() == rid).all()
                toks = sorted(rng.choice(w.t_decode, size=min(2, w.t_decode), replace=False))
                want = offn.moe_layer(tr.x_as_f32(x_bits), rid, rw, lambda e: src(l, e), w.wfmt,
                                      w.hidden, w.inter, tokens=toks)
                say(f"call ({s},{l}): hits {h['counts'][1]} fills {h['counts'][3]} "
                    f"in-place {h['counts'][4]}")
                check_close(got[toks], want, f"{w.name} call ({s},{l}) tokens {toks}")
