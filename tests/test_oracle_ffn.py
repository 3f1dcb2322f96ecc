"""Pins of the oracle's expert SwiGLU, combine and permutation: zero input,
hand-built experts with closed-form outputs (row-, column- and index-dependent
nibbles, so a transposed operand or a dropped term changes the answer), a
scalar-loop brute force that decodes the canonical bytes by index, and the
float32 path against the float64 one."""
import math

import numpy as np
import pytest

from oracle import ffn, formats
from workloads import experts as wx


def _bf16_bits(v):
    b = np.array([v], dtype=np.float32).view(np.uint32)[0]
    assert b & 0xFFFF == 0
    return int(b >> 16)


def _int4_matrix(nibble, s, b, out, inn):
    """Canonical bytes of one int4 matrix whose nibble at (o, i) is nibble(o, i)."""
    q = np.zeros(out * inn // 2, dtype=np.uint8)
    for o in range(out):
        for i in range(inn):
            v = nibble(o, i) & 0xF
            c = (o * inn + i) // 2
            q[c] |= np.uint8(v << (4 * (i % 2)))
    ng = out * inn // 64
    sb = np.full(ng, _bf16_bits(s), dtype=np.uint16)
    bb = np.full(ng, _bf16_bits(b), dtype=np.uint16)
    return [q, sb.view(np.uint8), bb.view(np.uint8)]


def _silu(z):
    if z >= 0:
        return z / (1.0 + math.exp(-z))
    e = math.exp(z)             # no overflow for large negative z
    return z * e / (1.0 + e)


def test_zero_input_gives_zero_output():
    H, I, E = 128, 64, 4
    blobs = {e: wx.expert_blob(9, e, formats.INT4_G64, H, I) for e in range(E)}
    x = np.zeros((3, H))
    ids = np.array([[0, 1], [2, 3], [1, 2]])
    w = np.full((3, 2), 0.5)
    out = ffn.moe_layer(x, ids, w, blobs.__getitem__, formats.INT4_G64, H, I)
    assert np.all(out == 0.0)


def _extreme_x(H):
    """Activations far outside N(0, 1): bf16 values of +-3e4 and +-7e4 (beyond
    f16's largest finite value) and +-1e-6 (below f16's normal range), mixed
    with ordinary ones."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, H))
    x[0, :6] = [3e4, -3e4, 7e4, -7e4, 1e-6, -1e-6]
    x[1, ::5] = 1e-6
    x[1, 1] = -7e4
    bits = (x.astype(np.float32).view(np.uint32) + 0x8000) >> 16      # bf16, nearest
    return formats.bf16_to_float(bits.astype(np.uint16))


@pytest.mark.parametrize("xkind", ["normal", "extreme"])
def test_closed_form_expert(xkind):
    H, I = 128, 64
    s0, b0, s1, b1, s2, b2 = 0.0078125, -0.03125, 0.015625, -0.0625, 0.00390625, -0.015625
    parts = (_int4_matrix(lambda o, i: o % 16, s0, b0, I, H)           # gate depends on the row
             + _int4_matrix(lambda o, i: i % 16, s1, b1, I, H)         # up depends on the column
             + _int4_matrix(lambda o, i: (o + 2 * i) % 16, s2, b2, H, I))
    blob = np.concatenate(parts)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((2, H)) if xkind == "normal" else _extreme_x(H)
    out = ffn.moe_layer(x, np.array([[0], [0]]), np.array([[1.0], [0.75]]),
                        lambda e: blob, formats.INT4_G64, H, I)
    for t, wt in ((0, 1.0), (1, 0.75)):
        sx = sum(x[t])
        cx = sum((c % 16) * x[t, c] for c in range(H))
        u = s1 * cx + b1 * sx                      # same for every row of up
        h = [_silu((s0 * (r % 16) + b0) * sx) * u for r in range(I)]
        for n in (0, 1, 17, H - 1):
            y = sum((s2 * ((n + 2 * i) % 16) + b2) * h[i] for i in range(I))
            assert abs(out[t, n] - wt * y) <= 1e-9 * max(1.0, abs(y))


def _nibble(blob, off, o, i, inn):
    byte = int(blob[off + (o * inn + i) // 2])
    return (byte >> (4 * (i % 2))) & 0xF


def _bf16_at(blob, off, idx):
    lo, hi = int(blob[off + 2 * idx]), int(blob[off + 2 * idx + 1])
    return float(np.array([(hi << 8 | lo) << 16], dtype=np.uint32).view(np.float32)[0])


def _brute_int4_weight(blob, H, I, m, o, i):
    """Weight (o, i) of matrix m (0 gate, 1 up, 2 down) read straight from the bytes."""
    dims = [(I, H), (I, H), (H, I)]
    off = 0
    for mm in range(m):
        out, inn = dims[mm]
        off += out * inn // 2 + 4 * (out * inn // 64)
    out, inn = dims[m]
    ng = out * inn // 64
    q = _nibble(blob, off, o, i, inn)
    g = o * (inn // 64) + i // 64
    s = _bf16_at(blob, off + out * inn // 2, g)
    b = _bf16_at(blob, off + out * inn // 2 + 2 * ng, g)
    return s * q + b


def _brute_mx_weight(blob, H, I, m, o, i):
    dims = [(I, H), (I, H), (H, I)]
    off = 0
    for mm in range(m):
        out, inn = dims[mm]
        off += out * inn // 2 + out * inn // 32
    out, inn = dims[m]
    code = _nibble(blob, off, o, i, inn)
    e = int(blob[off + out * inn // 2 + o * (inn // 32) + i // 32])
    sign = -1.0 if code & 8 else 1.0
    ex, man = (code >> 1) & 3, code & 1
    mag = 0.5 * man if ex == 0 else 2.0 ** (ex - 1) * (1 + 0.5 * man)
    return sign * mag * 2.0 ** (e - 127)


@pytest.mark.parametrize("wfmt", [formats.INT4_G64, formats.MXFP4])
def test_scalar_brute_force_tiny_layer(wfmt):
    H, I, E, T, k = 64, 64, 3, 3, 2
    blobs = {e: wx.expert_blob(17, e, wfmt, H, I) for e in range(E)}
    rng = np.random.default_rng(1)
    x = rng.standard_normal((T, H))
    ids = np.array([[0, 2], [1, 0], [2, 1]])
    w = rng.random((T, k))
    out = ffn.moe_layer(x, ids, w, blobs.__getitem__, wfmt, H, I)
    wt = _brute_int4_weight if wfmt == formats.INT4_G64 else _brute_mx_weight
    for t in range(T):
        acc = [0.0] * H
        for j in range(k):
            blob = blobs[int(ids[t, j])]
            g = [sum(wt(blob, H, I, 0, r, c) * x[t, c] for c in range(H)) for r in range(I)]
            u = [sum(wt(blob, H, I, 1, r, c) * x[t, c] for c in range(H)) for r in range(I)]
            h = [_silu(g[r]) * u[r] for r in range(I)]
            for n in range(H):
                acc[n] += w[t, j] * sum(wt(blob, H, I, 2, n, i) * h[i] for i in range(I))
        np.testing.assert_allclose(out[t], acc, rtol=1e-10, atol=1e-10)


def test_float32_path_within_float64_bound():
    H, I, E = 256, 128, 16
    blobs = {e: wx.expert_blob(1000, e, formats.INT4_G64, H, I) for e in range(E)}
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, H))
    ids = np.array([[0, 5], [3, 9], [15, 1], [7, 8]])
    w = np.array([[0.6, 0.4], [0.5, 0.5], [0.9, 0.1], [0.3, 0.7]])
    o64 = ffn.moe_layer(x, ids, w, blobs.__getitem__, formats.INT4_G64, H, I, dtype=np.float64)
    o32 = ffn.moe_layer(x, ids, w, blobs.__getitem__, formats.INT4_G64, H, I, dtype=np.float32)
    err = np.abs(o32 - o64).max()
    assert err < 1e-3 * max(1.0, np.abs(o64).max())


def test_token_subset_equals_full_rows():
    H, I, E = 128, 64, 8
    blobs = {e: wx.expert_blob(3, e, formats.MXFP4, H, I) for e in range(E)}
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, H))
    ids = np.stack([rng.choice(E, 3, replace=False) for _ in range(6)])
    w = rng.random((6, 3))
    full = ffn.moe_layer(x, ids, w, blobs.__getitem__, formats.MXFP4, H, I)
    sub = ffn.moe_layer(x, ids, w, blobs.__getitem__, formats.MXFP4, H, I, tokens=[4, 1])
    # BLAS may block a 2-row product differently from a 6-row one
    np.testing.assert_allclose(sub, full[[4, 1]], rtol=1e-10, atol=1e-15)


def test_permute_brute_force():
    rng = np.random.default_rng(6)
    E, T, k = 16, 50, 3
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    perm, offsets = ffn.permute(ids, E)
    want = [t * k + j for e in range(E) for t in range(T) for j in range(k) if ids[t, j] == e]
    assert perm.tolist() == want
    assert offsets[0] == 0 and offsets[-1] == T * k
    for e in range(E):
        assert offsets[e + 1] - offsets[e] == int((ids == e).sum())


def test_combine_hand_example():
    """Two tokens, three slots, small integers: every product and sum is exact."""
    y = np.array([[[1.0, 2.0], [10.0, 20.0], [100.0, 200.0]],
                  [[-1.0, 0.5], [4.0, -8.0], [0.0, 3.0]]])
    w = np.array([[0.5, 0.25, 0.125], [2.0, 0.0, 1.0]])
    out = ffn.combine(y, w)
    assert out.tolist() == [[0.5 + 2.5 + 12.5, 1.0 + 5.0 + 25.0], [-2.0, 1.0 + 3.0]]
    # one slot with weight 1 is the identity; a zero weight drops its slot
    assert np.array_equal(ffn.combine(y[:, :1], np.ones((2, 1))), y[:, 0])
    w2 = w.copy()
    w2[:, 1] = 0.0
    assert np.array_equal(ffn.combine(y, w2), ffn.combine(y[:, [0, 2]], w[:, [0, 2]]))
