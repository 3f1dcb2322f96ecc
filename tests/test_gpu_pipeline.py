"""Whole-layer buffered prefill over consecutive layers with the experts
streamed from a pinned host pool (moe355_prefill_layers), with two buffers
(copy of layer l+1 overlapping the compute of layer l) and with one: every
layer's output against the oracle, and the buffers holding the last layers'
pool bytes afterwards."""
import numpy as np
import pytest

from oracle import route as oroute
from workloads import configs as C
from workloads import experts as wx
from workloads import traces as tr

from gpu_common import BlobSource, ParityLog, desc_of, oracle_layer, packer, say

pytestmark = pytest.mark.gpu

SHAPES = [
    C.Workload(cid=190, name="pipe_int4", hidden=1024, inter=256, n_experts=16, top_k=2, route=0,
               wfmt=C.WFMT_INT4_G64, n_layers=5, t_prefill=300),
    C.Workload(cid=191, name="pipe_mxfp4", hidden=2048, inter=512, n_experts=16, top_k=3,
               route=C.ROUTE_SIGMOID_GROUP, n_group=4, topk_group=2, route_scale=2.5,
               wfmt=C.WFMT_MXFP4, n_layers=4, t_prefill=200),
]


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_prefill_layers_matches_oracle(w):
    import torch
    import moe_expert_layer_02_amd as m
    from workloads import gpu as wg
    desc = desc_of(w)
    L, T, E = w.n_layers, w.t_prefill, w.n_experts
    S = wx.expert_bytes(w.wfmt, w.hidden, w.inter)
    pool_dev = wg.make_pool(w, pack=packer(desc))
    host_pool = torch.empty(pool_dev.numel(), dtype=torch.uint8, pin_memory=True)
    host_pool.copy_(pool_dev)
    logits = [torch.from_numpy(tr.prefill_logits_layer(w, l)).cuda() for l in range(L)]
    xb = [tr.prefill_x_layer(w, l) for l in range(L)]
    xs = [torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16) for b in xb]
    bufs = [torch.empty(E * S, dtype=torch.uint8, device="cuda") for _ in range(2)]
    ids = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, w.top_k), dtype=torch.float32, device="cuda")
    perm = torch.empty(T * w.top_k, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    ws = torch.empty(m.workspace_bytes(desc, T, m.MODE_PREFILL), dtype=torch.uint8, device="cuda")
    wsp = torch.empty(m.workspace_bytes(desc, T, m.MODE_PERMUTE), dtype=torch.uint8, device="cuda")
    copy = torch.cuda.Stream()
    src = BlobSource(w)
    wants = []
    for l in range(L):
        rid, rw = oroute.route(tr.prefill_logits_layer(w, l), w.top_k, w.route, w.n_group,
                               w.topk_group, w.route_scale)
        wants.append(oracle_layer(tr.x_as_f32(xb[l]), rid, rw, lambda e, l=l: src(l, e), w.wfmt,
                                  w.hidden, w.inter))
    for double in (True, False):
        outs = [torch.full((T, w.hidden), float("nan"), dtype=torch.float32, device="cuda")
                for _ in range(L)]
        for b in bufs:
            b.fill_(0)
        m.prefill_layers(desc, host_pool, bufs, logits, xs, outs, ids, wt, perm, offsets, ws, wsp,
                         double, copy_stream=copy)
        torch.cuda.current_stream().wait_stream(copy)
        torch.cuda.synchronize()
        assert m.error_word(ws, m.MODE_PREFILL) == 0
        log = ParityLog(f"{w.name} {'two buffers' if double else 'one buffer'}")
        for l in range(L):
            log.check(outs[l].cpu().numpy(), wants[l], f"layer {l}")
        log.report()
        last = [L - 1, L - 2] if double else [L - 1]
        for l in last:
            b = bufs[l % 2] if double else bufs[0]
            assert torch.equal(b, pool_dev[l * E * S:(l + 1) * E * S]), f"buffer of layer {l}"
    say(f"{w.name}: {L} layers through one and two buffers match the oracle")


def test_prefill_layers_rejects_device_pool():
    import torch
    import moe_expert_layer_02_amd as m
    w = SHAPES[0]
    desc = desc_of(w)
    dev = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        m.prefill_layers(desc, dev, [dev, dev], [dev], [dev], [dev], dev, dev, dev, dev, dev, dev,
                         True, copy_stream=torch.cuda.Stream())
