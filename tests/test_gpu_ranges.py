"""The unfused combine call against the oracle's combine, and the activation
range contract of the expert FFN calls.

The int4 path runs its products on f16 operands (exact inside f16's range); an
activation beyond f16's finite range, or an intermediate h that leaves it,
must be reported through the call's error word, never passed off as a valid
output.  Tiny activations (1e-6, below f16's normal range) and moderately large
ones stay within the parity bar.  MXFP4 runs on bf16 operands: activations of
+-3e4 and +-7e4 are computed, with outputs near 1e8 checked to rel L2 1e-2 and
a max-abs bound scaled to the output (1e-4 of its largest magnitude: the hi/lo
bf16 split of h keeps about 16 significant bits, fp32 accumulation about 24)."""
import numpy as np
import pytest

from oracle import ffn as offn
from oracle import route as oroute
from workloads import configs as C
from workloads import experts as wx
from workloads import traces as tr

from gpu_common import BlobSource, check_close, desc_of, oracle_layer, packer, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,H,k", [(1, 4096, 8), (37, 2048, 6), (1000, 256, 1), (5, 4096, 2)])
def test_combine_matches_oracle(T, H, k):
    import torch
    import moe_expert_layer_02_amd as m
    rng = np.random.default_rng(T * 7 + H + k)
    y = (rng.standard_normal((T * k, H)) * 50).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    out = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    m.combine(torch.from_numpy(y).cuda(), torch.from_numpy(w).cuda(), out)
    torch.cuda.synchronize()
    want = offn.combine(y.reshape(T, k, H).astype(np.float64), w.astype(np.float64))
    got = out.cpu().numpy()
    # fp32 fused multiply-adds over k terms of magnitude <= ~250
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-4)
    say(f"combine T={T} H={H} k={k}: max abs err {np.abs(got - want).max():.2e}")


def test_combine_empty_batch():
    import torch
    import moe_expert_layer_02_amd as m
    y = torch.zeros((0, 64), dtype=torch.float32, device="cuda")
    w = torch.zeros((0, 2), dtype=torch.float32, device="cuda")
    out = torch.zeros((0, 64), dtype=torch.float32, device="cuda")
    m.combine(y, w, out)
    torch.cuda.synchronize()


def _x_case(kind, T, H, rng):
    """bf16 bits [T, H]: N(0, 1) with planted values."""
    x = rng.standard_normal((T, H)).astype(np.float32)
    if kind == "tiny_and_moderate":
        x[:, ::7] = 1e-6
        x[:, 3::11] = -3e-7
        x[0, 1:4] = [60.0, -45.0, 30.0]
    elif kind == "x_beyond_f16":
        x[T - 1, 5] = 7.0e4
        x[0, 9] = -7.0e4
    elif kind == "h_beyond_f16":      # x fits f16, silu(g) * u does not
        x[0, 2] = 3.0e4
        x[T - 1, 7] = -3.0e4
    return wx.f32_to_bf16_bits(x)


def _route(E, k, T, rng):
    logits = rng.standard_normal((T, E)).astype(np.float32)
    return oroute.softmax_topk(logits, k)


def _check(kind, wfmt, got, want, err, what):
    import moe_expert_layer_02_amd as m
    if wfmt == C.WFMT_INT4_G64 and kind != "tiny_and_moderate":
        assert err & m.ERR_F16_RANGE, f"{what}: out-of-range input not flagged (error word {err:#x})"
        say(f"{what}: flagged (error word {err:#x})")
        return
    assert err == 0, f"{what}: error word {err:#x}"
    if kind == "tiny_and_moderate":
        check_close(got, want, what)
        return
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    mx = np.abs(got - want).max()
    say(f"{what}: rel_l2={rel:.3e} max_abs={mx:.3e} (|ref| max {np.abs(want).max():.3e})")
    assert np.all(np.isfinite(got)) and rel <= 1e-2 and mx <= 1e-4 * np.abs(want).max()


KINDS = ["tiny_and_moderate", "x_beyond_f16", "h_beyond_f16"]


@pytest.mark.parametrize("T", [3, 20])          # one-launch small call; two launches
@pytest.mark.parametrize("wfmt", [C.WFMT_INT4_G64, C.WFMT_MXFP4])
@pytest.mark.parametrize("kind", KINDS)
def test_decode_activation_range(kind, wfmt, T):
    import torch
    import moe_expert_layer_02_amd as m
    from workloads import gpu as wg
    w = C.Workload(cid=150 + wfmt, name="range", hidden=1024, inter=256, n_experts=8, top_k=2,
                   route=0, wfmt=wfmt)
    rng = np.random.default_rng(T + 31 * wfmt + len(kind))
    desc = desc_of(w)
    x_bits = _x_case(kind, T, w.hidden, rng)
    ids_np, wt_np = _route(w.n_experts, w.top_k, T, rng)
    layer = wg.make_experts(w, 0, w.n_experts, C.seed(w.cid, 0), pack=packer(desc))
    ids = torch.from_numpy(ids_np.astype(np.int32)).cuda()
    wt = torch.from_numpy(wt_np.astype(np.float32)).cuda()
    exp = m.DeviceClassifyOut(min(T * w.top_k, w.n_experts))
    m.dedup(ids, w.n_experts, exp)
    out = torch.full((T, w.hidden), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros(m.workspace_bytes(desc, T, m.MODE_DECODE), dtype=torch.uint8, device="cuda")
    xd = torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    m.expert_ffn_decode(desc, xd, ids, wt, None, layer, 0, exp, out, ws)
    torch.cuda.synchronize()
    err = m.error_word(ws)
    src = BlobSource(w)
    want = oracle_layer(tr.x_as_f32(x_bits), ids_np, wt_np, lambda e: src(0, e), wfmt,
                        w.hidden, w.inter)
    _check(kind, wfmt, out.cpu().numpy().astype(np.float64), want, err,
           f"decode {kind} fmt={wfmt} T={T}")


@pytest.mark.parametrize("wfmt", [C.WFMT_INT4_G64, C.WFMT_MXFP4])
@pytest.mark.parametrize("kind", KINDS)
def test_prefill_activation_range(kind, wfmt):
    """Also: the prefill error word is cleared by the next call."""
    import torch
    import moe_expert_layer_02_amd as m
    from workloads import gpu as wg
    w = C.Workload(cid=160 + wfmt, name="range-pf", hidden=1024, inter=256, n_experts=8,
                   top_k=2, route=0, wfmt=wfmt)
    T = 300
    rng = np.random.default_rng(97 + wfmt + len(kind))
    desc = desc_of(w)
    layer = wg.make_experts(w, 0, w.n_experts, C.seed(w.cid, 0), pack=packer(desc))
    ws = torch.empty(m.workspace_bytes(desc, T, m.MODE_PREFILL), dtype=torch.uint8, device="cuda")
    wsp = torch.empty(m.workspace_bytes(desc, T, m.MODE_PERMUTE), dtype=torch.uint8, device="cuda")
    ws[:4].fill_(0xFF)      # a stale word from an earlier call
    src = BlobSource(w)
    for case in (kind, "tiny_and_moderate"):
        x_bits = _x_case(case, T, w.hidden, rng)
        ids_np, wt_np = _route(w.n_experts, w.top_k, T, rng)
        ids = torch.from_numpy(ids_np.astype(np.int32)).cuda()
        wt = torch.from_numpy(wt_np.astype(np.float32)).cuda()
        perm = torch.empty(T * w.top_k, dtype=torch.int32, device="cuda")
        offsets = torch.empty(w.n_experts + 1, dtype=torch.int32, device="cuda")
        m.permute(desc, ids, perm, offsets, wsp)
        out = torch.full((T, w.hidden), float("nan"), dtype=torch.float32, device="cuda")
        xd = torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)
        m.expert_ffn_prefill(desc, xd, ids, wt, layer, perm, offsets, out, ws)
        torch.cuda.synchronize()
        err = m.error_word(ws, m.MODE_PREFILL)
        want = oracle_layer(tr.x_as_f32(x_bits), ids_np, wt_np, lambda e: src(0, e), wfmt,
                            w.hidden, w.inter)
        _check(case, wfmt, out.cpu().numpy().astype(np.float64), want, err,
               f"prefill {case} fmt={wfmt}")
