"""Pins of the oracle's MX FP8 E4M3 activation quantisation (OCP Microscaling
Formats v1.0) and of the layer over MXFP4 experts with MX activations:
hand-built blocks with known shared exponents, ties, saturation and
subnormals; an exhaustive search over the 254 finite E4M3 codes (nearest value,
ties to the even code) and over the shared exponents that replaces the
closed forms; and a scalar-loop brute force of a tiny MX layer."""
import math

import numpy as np
import pytest

from oracle import ffn, formats
from workloads import experts as wx

from test_oracle_ffn import _brute_mx_weight, _silu

FINITE = [c for c in range(256) if c not in (0x7F, 0xFF)]


def test_e4m3_code_table():
    vals = {c: formats.e4m3_value(c) for c in FINITE}
    assert vals[0x00] == 0.0 and vals[0x01] == 2.0 ** -9 and vals[0x07] == 7 * 2.0 ** -9
    assert vals[0x08] == 2.0 ** -6 and vals[0x38] == 1.0 and vals[0x78] == 256.0
    assert vals[0x7E] == 448.0 and vals[0xFE] == -448.0 and vals[0xB8] == -1.0
    assert math.isnan(formats.e4m3_value(0x7F)) and math.isnan(formats.e4m3_value(0xFF))
    pos = sorted(v for c, v in vals.items() if c < 0x80)
    assert len(set(pos)) == 127 and max(pos) == 448.0


def _block(vals):
    b = np.zeros(32)
    b[:len(vals)] = vals
    return b


def test_hand_built_blocks():
    # amax 1 -> e = 0 - 8: 1.0 is stored as 256 * 2**-8, code 0x78, scale byte 119
    q, s = formats.mx_quantize(_block([1.0, -0.5]))
    assert s.tolist() == [119] and q[0] == 0x78 and q[1] == 0xF0
    # amax 256 -> e = 0: spacing 2 in [16, 32): 17 ties to 16 (even), 19 to 20, 18 stays
    q, s = formats.mx_quantize(_block([256.0, 17.0, 19.0, 18.0, -17.0]))
    assert s.tolist() == [127]
    assert [formats.e4m3_value(c) for c in q[:5]] == [256.0, 16.0, 20.0, 18.0, -16.0]
    # amax 500 -> e = 0: 500 saturates to 448, 460 rounds to 448, 470 would round to 480
    q, _ = formats.mx_quantize(_block([500.0, 460.0, 470.0, -1000.0 / 2.0]))
    assert [formats.e4m3_value(c) for c in q[:4]] == [448.0, 448.0, 448.0, -448.0]
    # subnormals at e = 0: 3 * 2**-9 exact, 2**-10 ties to 0, 1.5 * 2**-9 ties to 2 * 2**-9
    q, _ = formats.mx_quantize(_block([256.0, 3 * 2.0 ** -9, 2.0 ** -10, 1.5 * 2.0 ** -9]))
    assert q[1] == 0x03 and q[2] == 0x00 and q[3] == 0x02
    # a zero block takes the smallest scale; zeros and negative zeros are +0
    q, s = formats.mx_quantize(np.array([0.0, -0.0] * 16))
    assert s.tolist() == [0] and not q.any()
    q, _ = formats.mx_quantize(_block([1.0, -2.0 ** -30]))
    assert q[1] == 0x00
    # the shared exponent follows amax across binades and clamps to e8m0's range
    for amax, e in ((1.0, -8), (1.99, -8), (2.0, -7), (3e4, 6), (2.0 ** -140, -127), (2.0 ** 140, 127)):
        assert int(formats.mx_shared_exponent(np.array(amax))) == e, amax


def _nearest_code(v):
    """Exhaustive: the finite code nearest to v (clamped to +-448), ties to the even code."""
    v = min(max(v, -448.0), 448.0)
    best = None
    for c in FINITE:
        d = abs(formats.e4m3_value(c) - v)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
            best = (d, c)
    c = best[1]
    return 0 if formats.e4m3_value(c) == 0.0 else c


def _search_exponent(amax):
    """The largest e in [-127, 127] with 2**(e + 8) <= amax (scanning down), else -127."""
    for e in range(127, -128, -1):
        if 2.0 ** (e + 8) <= amax:
            return e
    return -127


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_quantiser_matches_exhaustive_search(seed):
    rng = np.random.default_rng(seed)
    scales = [1e-3, 1.0, 37.0, 3e4, 1e-38][seed::3] + [1.0]
    for sc in scales:
        v = rng.standard_normal(64) * sc
        v[rng.integers(0, 64, 4)] = 0.0
        q, s = formats.mx_quantize(v)
        for b in range(2):
            blk = v[32 * b:32 * b + 32]
            e = _search_exponent(np.abs(blk).max()) if np.abs(blk).max() > 0 else -127
            assert int(s[b]) == e + 127, (sc, b)
            for i in range(32):
                want = _nearest_code(math.ldexp(blk[i], -e))
                assert int(q[32 * b + i]) == want, (sc, b, i, blk[i])


def test_round_trip_error_and_idempotence():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((8, 256)) * np.exp(rng.uniform(-5, 5, (8, 1)))
    r = formats.mx_round_trip(v)
    # relative error of a normal element is at most half of 2**-3; subnormals are
    # within half the block's subnormal step; elements above 448 * 2**e saturate
    blocks = v.reshape(8, 8, 32)
    e = formats.mx_shared_exponent(np.abs(blocks).max(-1))[..., None]
    step_floor = np.ldexp(1.0, e - 9)
    sat = np.abs(blocks) - np.ldexp(448.0, e)
    err = np.abs(r.reshape(8, 8, 32) - blocks)
    bound = np.maximum(np.maximum(np.abs(blocks) * 2.0 ** -4, step_floor / 2), sat)
    assert np.all(err <= bound * (1 + 1e-12))
    assert np.any(sat > 0)      # the draw does reach the saturation band
    assert np.array_equal(formats.mx_round_trip(r), r)


def _brute_mx8(v):
    """Scalar MX round trip of a vector by exhaustive search (blocks of 32)."""
    out = []
    for b in range(0, len(v), 32):
        blk = v[b:b + 32]
        amax = max(abs(t) for t in blk)
        e = _search_exponent(amax) if amax > 0 else -127
        out += [formats.e4m3_value(_nearest_code(math.ldexp(t, -e))) * 2.0 ** e for t in blk]
    return out


def test_mx_layer_scalar_brute_force():
    H, I, E, T, k = 64, 64, 3, 2, 2
    blobs = {e: wx.expert_blob(23, e, formats.MXFP4, H, I) for e in range(E)}
    rng = np.random.default_rng(11)
    x = rng.standard_normal((T, H)) * 3
    ids = np.array([[0, 2], [2, 1]])
    w = rng.random((T, k))
    out = ffn.moe_layer_mx8(x, ids, w, blobs.__getitem__, H, I)
    for t in range(T):
        xq = _brute_mx8(list(x[t]))
        acc = [0.0] * H
        for j in range(k):
            blob = blobs[int(ids[t, j])]
            g = [sum(_brute_mx_weight(blob, H, I, 0, r, c) * xq[c] for c in range(H)) for r in range(I)]
            u = [sum(_brute_mx_weight(blob, H, I, 1, r, c) * xq[c] for c in range(H)) for r in range(I)]
            h = [_silu(g[r]) * u[r] for r in range(I)]
            h1 = _brute_mx8(h)
            h2 = _brute_mx8([a - b for a, b in zip(h, h1)])
            for n in range(H):
                acc[n] += w[t, j] * sum(_brute_mx_weight(blob, H, I, 2, n, i) * (h1[i] + h2[i])
                                        for i in range(I))
        np.testing.assert_allclose(out[t], acc, rtol=1e-10, atol=1e-12)


def test_mx_layer_close_to_plain_layer_on_quantised_x():
    """With x already on the MX grid, the only difference from the plain layer is
    h's two-term quantisation, whose error is at most half the second term's
    step: a quarter of 2**-3 of the first term's, relative to the block."""
    H, I, E = 256, 128, 8
    blobs = {e: wx.expert_blob(29, e, formats.MXFP4, H, I) for e in range(E)}
    rng = np.random.default_rng(12)
    x = formats.mx_round_trip(rng.standard_normal((5, H)))
    ids = np.stack([rng.choice(E, 2, replace=False) for _ in range(5)])
    w = rng.random((5, 2))
    a = ffn.moe_layer_mx8(x, ids, w, blobs.__getitem__, H, I)
    b = ffn.moe_layer(x, ids, w, blobs.__getitem__, formats.MXFP4, H, I)
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    assert 0 < rel < 2e-3, rel
    assert np.all(ffn.moe_layer_mx8(np.zeros((2, H)), ids[:2], w[:2], blobs.__getitem__, H, I) == 0)
