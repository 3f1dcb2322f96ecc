"""Prefill parity on the GPU: the expert permutation bit-exact against the
oracle's stable sort, and the grouped-GEMM expert FFN (route -> permute ->
expert_ffn_prefill) against the oracle on small shapes that span several
tiles with ragged buckets and empty experts, and on sampled tokens of the two
full-size prefill workloads."""
import numpy as np
import pytest

from oracle import ffn as offn
from oracle import route as oroute
from workloads import configs as C
from workloads import experts as wx
from workloads import traces as tr

from gpu_common import BlobSource, check_close, desc_of, oracle_layer, packer, say

pytestmark = pytest.mark.gpu


def _gpu_permute(w, ids_np):
    import torch
    import moe_expert_layer_02_amd as m
    desc = desc_of(w)
    T = ids_np.shape[0]
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).cuda()
    perm = torch.full((max(T * w.top_k, 1),), -7, dtype=torch.int32, device="cuda")
    offsets = torch.full((w.n_experts + 1,), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(m.workspace_bytes(desc, T, m.MODE_PERMUTE), dtype=torch.uint8, device="cuda")
    m.permute(desc, ids, perm, offsets, ws)
    torch.cuda.synchronize()
    return perm.cpu().numpy()[:T * w.top_k], offsets.cpu().numpy()


@pytest.mark.parametrize("E,k,T", [(16, 2, 4), (256, 8, 8192), (256, 6, 16384), (64, 3, 1000),
                                   (1024, 4, 777), (8, 8, 3000)])
def test_permute_matches_oracle(E, k, T):
    w = C.Workload(cid=130, name="perm", hidden=256, inter=128, n_experts=E, top_k=k, route=0)
    rng = np.random.default_rng(E + k + T)
    # skewed routing, with some experts left empty
    pop = rng.random(E) ** 4
    n_empty = min(E // 8, E - k)
    pop[rng.choice(E, size=n_empty, replace=False)] = 0
    pop /= pop.sum()
    ids = np.stack([rng.choice(E, size=k, replace=False, p=pop) for _ in range(T)]).astype(np.int32)
    perm, offsets = _gpu_permute(w, ids)
    rperm, roff = offn.permute(ids, E)
    assert np.array_equal(offsets, roff)
    assert np.array_equal(perm, rperm)


def _prefill(w, x_bits, ids_np, wt_np, layer_seed, with_err=False):
    import torch
    import moe_expert_layer_02_amd as m
    from workloads import gpu as wg
    desc = desc_of(w)
    T = x_bits.shape[0]
    S = wx.expert_bytes(w.wfmt, w.hidden, w.inter)
    layer = wg.make_experts(w, 0, w.n_experts, layer_seed, pack=packer(desc))
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).cuda()
    wt = torch.from_numpy(np.ascontiguousarray(wt_np, dtype=np.float32)).cuda()
    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda().view(torch.bfloat16)
    perm = torch.empty(T * w.top_k, dtype=torch.int32, device="cuda")
    offsets = torch.empty(w.n_experts + 1, dtype=torch.int32, device="cuda")
    wsp = torch.empty(m.workspace_bytes(desc, T, m.MODE_PERMUTE), dtype=torch.uint8, device="cuda")
    m.permute(desc, ids, perm, offsets, wsp)
    out = torch.full((T, w.hidden), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(m.workspace_bytes(desc, T, m.MODE_PREFILL), dtype=torch.uint8, device="cuda")
    m.expert_ffn_prefill(desc, x, ids, wt, layer, perm, offsets, out, ws)
    torch.cuda.synchronize()
    if with_err:
        return out, m.error_word(ws, m.MODE_PREFILL)
    assert m.error_word(ws, m.MODE_PREFILL) == 0
    return out


SMALL = [
    # (H, I, E, k, T, wfmt): buckets from a few rows to several 128-row tiles
    (256, 128, 16, 2, 300, C.WFMT_INT4_G64),
    (1024, 256, 8, 2, 517, C.WFMT_INT4_G64),
    (2048, 512, 32, 4, 700, C.WFMT_INT4_G64),
    (512, 256, 16, 3, 450, C.WFMT_MXFP4),
    (4096, 2048, 8, 2, 260, C.WFMT_MXFP4),
    (4096, 1024, 12, 3, 333, C.WFMT_INT4_G64),
]


@pytest.mark.parametrize("H,I,E,k,T,wfmt", SMALL)
def test_prefill_small_shapes(H, I, E, k, T, wfmt):
    w = C.Workload(cid=140 + E, name="pf-small", hidden=H, inter=I, n_experts=E, top_k=k,
                   route=0, wfmt=wfmt)
    say(f"prefill small H={H} I={I} E={E} k={k} T={T} fmt={wfmt}")
    rng = np.random.default_rng(H + I + E + k + T)
    x_bits = tr.bf16_normal(rng, (T, H))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, E - 1] -= 100.0          # one expert never routed: an empty bucket
    ids, wt = oroute.softmax_topk(logits, k)
    out = _prefill(w, x_bits, ids, wt, C.seed(w.cid, 0)).cpu().numpy()
    src = BlobSource(w)
    want = offn.moe_layer(tr.x_as_f32(x_bits), ids, wt, lambda e: src(0, e), wfmt, H, I)
    check_close(out, want, f"prefill H={H} I={I} fmt={wfmt}")


def _tile_row_tokens(ids_np, E, k, experts, rows_in_tile):
    """Tokens whose pairs sit at the given rows of 128-row tiles of each listed
    expert's bucket (plus the bucket's last row), from the oracle's permutation."""
    perm, offsets = offn.permute(ids_np, E)
    toks = set()
    for e in experts:
        b, n = int(offsets[e]), int(offsets[e + 1] - offsets[e])
        for r in sorted({t0 + r for t0 in range(0, n, 128) for r in rows_in_tile} | {n - 1}):
            if 0 <= r < n:
                toks.add(int(perm[b + r]) // k)
    return np.array(sorted(toks))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cid", [3, 5])
def test_prefill_full_size_sampled(cid):
    """The full-size prefill layers, every output checked for finiteness and the
    error word clear, and many tokens checked against the oracle: for the
    Qwen-like layer the tokens at the first, middle and last row of every
    128-row tile of every expert's bucket (and each bucket's last row); for the
    DS-like layer the first and last row of every tile of every eighth expert."""
    import torch
    import moe_expert_layer_02_amd as m
    w = C.ALL[cid]
    T = w.t_prefill
    say(f"prefill full size {w.name}: T={T}")
    x_bits = tr.prefill_x(w)
    logits = tr.prefill_logits(w)
    # route on the GPU (bit-exact ids are checked in the router tests)
    desc = desc_of(w)
    lg = torch.from_numpy(logits).cuda()
    ids = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, w.top_k), dtype=torch.float32, device="cuda")
    m.route(desc, lg, ids, wt)
    torch.cuda.synchronize()
    ids_np, wt_np = ids.cpu().numpy(), wt.cpu().numpy()
    counts = np.bincount(ids_np.ravel(), minlength=w.n_experts)
    say(f"tokens per expert: min {counts.min()} max {counts.max()}")
    assert counts.min() > 0
    out, err = _prefill(w, x_bits, ids_np, wt_np, C.seed(w.cid, 0), with_err=True)
    assert err == 0, f"error word {err:#x}"
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    experts = range(w.n_experts) if cid == 3 else range(0, w.n_experts, 8)
    rows = (0, 63, 64, 127) if cid == 3 else (0, 127)
    toks = _tile_row_tokens(ids_np, w.n_experts, w.top_k, experts, rows)
    toks = np.union1d(toks, [0, T - 1])
    hit = np.unique(ids_np[toks])
    say(f"{len(toks)} tokens checked, covering {len(hit)} experts")
    assert len(toks) >= (512 if cid == 3 else 64)
    if cid == 3:
        assert len(hit) == w.n_experts
    src = BlobSource(w)
    rid, rw = oroute.route(logits[toks], w.top_k, w.route, w.n_group, w.topk_group, w.route_scale)
    assert np.array_equal(rid, ids_np[toks])
    want = oracle_layer(tr.x_as_f32(x_bits[toks]), rid, rw, lambda e: src(0, e), w.wfmt,
                        w.hidden, w.inter)
    check_close(got[toks], want, f"{w.name} {len(toks)} tokens")
