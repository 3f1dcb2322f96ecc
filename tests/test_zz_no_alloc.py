"""The allocation-free decode layer call (moe355_decode_layer_static, the
library's fixed per-GPU scratch in place of a workspace) against the workspace
form (moe355_decode_layer) through the C ABI: two calls in a row on the same
inputs and separate, identical caches, the second with fewer tokens; routing,
every list, the cache state and the layer output must agree (integers
bit-exact, outputs within the parity bar), and the error word stays clear.
Shapes: a small call (one launch) and a DS-like call (bookkeeping kernel, then
the two-launch FFN with h in the scratch)."""
import numpy as np
import pytest

from workloads import configs as C
from workloads import experts as wx
from workloads import traces as tr

from gpu_common import check_close, desc_of, packer, say

pytestmark = pytest.mark.gpu

SHAPES = {
    "small_int4": C.Workload(cid=170, name="static_small_int4", hidden=1024, inter=256,
                             n_experts=32, top_k=4, route=C.ROUTE_SOFTMAX_TOPK,
                             wfmt=C.WFMT_INT4_G64, n_layers=2, n_slots=24, t_decode=3, steps=2,
                             zipf_alpha=1.1, keep_prob=0.5, q_num=2, q_den=3),
    "ds_mxfp4": C.Workload(cid=171, name="static_ds_mxfp4", hidden=2048, inter=512,
                           n_experts=64, top_k=6, route=C.ROUTE_SIGMOID_GROUP, n_group=8,
                           topk_group=4, route_scale=2.5, wfmt=C.WFMT_MXFP4, n_layers=2,
                           n_slots=80, t_decode=16, steps=2, zipf_alpha=1.0, keep_prob=0.6),
}


@pytest.mark.parametrize("shape", list(SHAPES))
def test_static_scratch_matches_workspace_form(shape):
    import torch
    import moe_expert_layer_02_amd as m
    from workloads import gpu as wg
    w = SHAPES[shape]
    desc = desc_of(w)
    S = wx.expert_bytes(w.wfmt, w.hidden, w.inter)
    pool = wg.make_pool(w, pack=packer(desc))
    trace = tr.DecodeTrace(w, 2)
    K = min(w.t_decode * w.top_k, w.n_experts, w.n_slots)
    policy = m.EvictPolicy(K, w.q_num, w.q_den)
    cap = max(K, min(w.t_decode * w.top_k, w.n_experts))
    caches = [m.DeviceCache(w.n_slots, w.n_layers, w.n_experts, S) for _ in range(2)]
    ws = torch.zeros(m.workspace_bytes(desc, w.t_decode, m.MODE_DECODE), dtype=torch.uint8,
                     device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    # two calls in a row: all tokens of layer 0, then fewer tokens of layer 1
    for call, (layer, T) in enumerate(((0, w.t_decode), (1, max(1, w.t_decode // 3)))):
        say(f"{w.name}: call {call}, layer {layer}, T={T}")
        logits = torch.from_numpy(np.ascontiguousarray(trace.logits[call, layer, :T])).cuda()
        xb = tr.decode_x(w, call, layer)[:T]
        x = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).cuda().view(torch.bfloat16)
        res = []
        for form, cache in zip(("workspace", "static"), caches):
            ids = torch.full((T, w.top_k), -1, dtype=torch.int32, device="cuda")
            wt = torch.full((T, w.top_k), float("nan"), dtype=torch.float32, device="cuda")
            lists = m.DeviceClassifyOut(cap)
            out = torch.full((T, w.hidden), float("nan"), dtype=torch.float32, device="cuda")
            if form == "workspace":
                m.decode_layer(desc, cache, pool, layer, None, call + 1, logits, x, policy, ids, wt,
                               lists, out, ws)
            else:
                m.decode_layer_static(desc, cache, pool, layer, None, call + 1, logits, x, policy,
                                      ids, wt, lists, out, err)
            torch.cuda.synchronize()
            res.append((ids.cpu().numpy(), wt.cpu().numpy(), lists.host(), out.cpu().numpy()))
        m.check_error(ws, what=f"{w.name} workspace form")
        assert int(err.item()) == 0, f"static form error word {int(err.item()):#x}"
        (ia, wa, la, oa), (ib, wb, lb, ob) = res
        assert np.array_equal(ia, ib) and np.array_equal(wa.view(np.int32), wb.view(np.int32))
        for key in ("uniq", "hit_expert", "hit_slot", "miss", "fill_expert", "fill_slot",
                    "inplace", "victims", "counts", "plan"):
            assert la[key] == lb[key], (call, key)
        for a, b in zip((caches[0].table, caches[0].owner, caches[0].ts),
                        (caches[1].table, caches[1].owner, caches[1].ts)):
            assert torch.equal(a, b), call
        occ = torch.nonzero(caches[0].owner >= 0).flatten()
        assert occ.numel() > 0
        assert torch.equal(caches[0].data.view(-1, S).index_select(0, occ),
                           caches[1].data.view(-1, S).index_select(0, occ)), call
        check_close(ob, oa, f"{w.name} call {call} (T={T}) static vs workspace")
    say(f"{w.name}: static scratch form matches the workspace form on two calls")
