"""The native fp4 matrix-core prefill path (MXFP4 weights x MX FP8 E4M3
activations) on the GPU: the activation quantiser byte-exact against the
oracle's (codes and scale bytes, including ties, saturation, subnormals, zero
blocks and extreme bf16 magnitudes), and the MX expert FFN against the oracle's
layer on the same quantised operands (``ffn.moe_layer_mx8``) at the parity
bar, on small shapes with ragged and empty buckets and on tokens at the first
and last rows of the tiles of the DS-like prefill layer.  The MX result's
distance from the unquantised layer is reported, not asserted beyond a sanity
bound (that is the quantisation of x, not an error)."""
import numpy as np
import pytest

from oracle import ffn as offn
from oracle import formats
from oracle import route as oroute
from workloads import configs as C
from workloads import experts as wx
from workloads import traces as tr

from gpu_common import BlobSource, check_close, desc_of, oracle_layer, packer, say

pytestmark = pytest.mark.gpu


def _quantize_gpu(x_bits):
    import torch
    import moe_expert_layer_02_amd as m
    rows, cols = x_bits.shape
    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda().view(torch.bfloat16)
    codes = torch.full((rows, cols), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((rows, cols // 32), 0xAB, dtype=torch.uint8, device="cuda")
    m.quantize_mx(x, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def _special_rows(cols, rng):
    """bf16 rows with ties, saturation, subnormal elements, zeros and extremes."""
    rows = []
    r = np.zeros(cols, dtype=np.float32)
    r[:5] = [256.0, 17.0, 19.0, 18.0, -17.0]           # ties at spacing 2
    r[32:36] = [500.0, 460.0, 470.0, -480.0]            # saturation band
    r[64:68] = [256.0, 3 * 2.0 ** -9, 2.0 ** -10, 1.5 * 2.0 ** -9]   # subnormal elements
    r[96] = -0.0                                        # a block of (negative) zeros
    rows.append(r)
    big = rng.standard_normal(cols).astype(np.float32)
    big[::9] = 3.0e38                                   # near bf16's largest finite value
    big[1::9] = -2.0e38
    rows.append(big)
    tiny = (rng.standard_normal(cols) * 1e-39).astype(np.float32)   # bf16 subnormals
    rows.append(tiny)
    rows.append((rng.standard_normal(cols) * 1e-3).astype(np.float32))
    return wx.f32_to_bf16_bits(np.stack(rows))


@pytest.mark.parametrize("rows,cols", [(4, 128), (37, 4096), (1000, 256)])
def test_quantize_mx_bit_exact(rows, cols):
    rng = np.random.default_rng(rows + cols)
    x_bits = tr.bf16_normal(rng, (rows, cols))
    x_bits[:4] = _special_rows(cols, rng)
    got_c, got_s = _quantize_gpu(x_bits)
    want_c, want_s = formats.mx_quantize(tr.x_as_f32(x_bits).astype(np.float64))
    bad = np.nonzero(got_c != want_c)
    assert np.array_equal(got_s, want_s), np.nonzero(got_s != want_s)
    assert bad[0].size == 0, (bad[0][:5], bad[1][:5], got_c[bad][:5], want_c[bad][:5])
    say(f"quantize_mx {rows}x{cols}: codes and scales byte-exact")


def _mx_prefill(w, x_bits, ids_np, wt_np, layer_seed):
    import torch
    import moe_expert_layer_02_amd as m
    from workloads import gpu as wg
    desc = desc_of(w)
    T = x_bits.shape[0]
    layer = wg.make_experts(w, 0, w.n_experts, layer_seed, pack=packer(desc))
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).cuda()
    wt = torch.from_numpy(np.ascontiguousarray(wt_np, dtype=np.float32)).cuda()
    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda().view(torch.bfloat16)
    perm = torch.empty(T * w.top_k, dtype=torch.int32, device="cuda")
    offsets = torch.empty(w.n_experts + 1, dtype=torch.int32, device="cuda")
    wsp = torch.empty(m.workspace_bytes(desc, T, m.MODE_PERMUTE), dtype=torch.uint8, device="cuda")
    m.permute(desc, ids, perm, offsets, wsp)
    out = torch.full((T, w.hidden), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(m.workspace_bytes(desc, T, m.MODE_PREFILL_MX), dtype=torch.uint8,
                     device="cuda")
    ws[:4].fill_(0xFF)
    m.expert_ffn_prefill_mx(desc, x, ids, wt, layer, perm, offsets, out, ws)
    torch.cuda.synchronize()
    assert m.error_word(ws, m.MODE_PREFILL) == 0
    return out.cpu().numpy()


def _oracle_mx(w, x_bits, ids, wt, tokens=None):
    src = BlobSource(w)
    return offn.moe_layer_mx8(tr.x_as_f32(x_bits), ids, wt, lambda e: src(0, e), w.hidden,
                              w.inter, tokens=tokens)


SMALL = [
    # (H, I, E, k, T): buckets from a few rows to several 128-row tiles
    (256, 128, 16, 2, 300),
    (512, 256, 16, 3, 450),
    (1024, 512, 8, 2, 517),
    (4096, 2048, 8, 2, 260),
    (2048, 384, 12, 3, 333),
]


@pytest.mark.parametrize("H,I,E,k,T", SMALL)
def test_prefill_mx_small_shapes(H, I, E, k, T):
    w = C.Workload(cid=180 + E, name="pf-mx", hidden=H, inter=I, n_experts=E, top_k=k, route=0,
                   wfmt=C.WFMT_MXFP4)
    say(f"prefill mx H={H} I={I} E={E} k={k} T={T}")
    rng = np.random.default_rng(H + I + E + k + T)
    x_bits = tr.bf16_normal(rng, (T, H))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, E - 1] -= 100.0          # one expert never routed: an empty bucket
    ids, wt = oroute.softmax_topk(logits, k)
    got = _mx_prefill(w, x_bits, ids, wt, C.seed(w.cid, 0))
    want = _oracle_mx(w, x_bits, ids, wt)
    check_close(got, want, f"prefill mx H={H} I={I} against the MX oracle")
    src = BlobSource(w)
    plain = offn.moe_layer(tr.x_as_f32(x_bits), ids, wt, lambda e: src(0, e), C.WFMT_MXFP4, H, I)
    rel = np.linalg.norm(got - plain) / np.linalg.norm(plain)
    say(f"  distance from the unquantised layer: rel_l2={rel:.3e}")
    assert rel < 0.2


@pytest.mark.timeout(900)
def test_prefill_mx_full_size_sampled():
    """The DS-like prefill layer (T=16384, H=4096, I=2048, E=256, k=6) on the MX
    path: every output finite, and the tokens at the first and last row of every
    tile of every eighth expert's bucket against the MX oracle."""
    import torch
    import moe_expert_layer_02_amd as m
    from test_gpu_prefill import _tile_row_tokens
    w = C.DS_STRESS
    T = w.t_prefill
    x_bits = tr.prefill_x(w)
    logits = tr.prefill_logits(w)
    desc = desc_of(w)
    ids = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, w.top_k), dtype=torch.float32, device="cuda")
    m.route(desc, torch.from_numpy(logits).cuda(), ids, wt)
    torch.cuda.synchronize()
    ids_np, wt_np = ids.cpu().numpy(), wt.cpu().numpy()
    got = _mx_prefill(w, x_bits, ids_np, wt_np, C.seed(w.cid, 0))
    assert np.all(np.isfinite(got))
    toks = _tile_row_tokens(ids_np, w.n_experts, w.top_k, range(0, w.n_experts, 8), (0, 127))
    toks = np.union1d(toks, [0, T - 1])
    say(f"{len(toks)} tokens checked")
    assert len(toks) >= 64
    rid, rw = oroute.route(logits[toks], w.top_k, w.route, w.n_group, w.topk_group, w.route_scale)
    assert np.array_equal(rid, ids_np[toks])
    src = BlobSource(w)
    want = oracle_layer(tr.x_as_f32(x_bits[toks]), rid, rw, lambda e: src(0, e), w.wfmt,
                        w.hidden, w.inter, mx=True)
    check_close(got[toks], want, f"{w.name} MX path, {len(toks)} tokens")
