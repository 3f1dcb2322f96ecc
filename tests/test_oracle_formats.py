"""Pins of the oracle's weight decoding against hand-built bytes, the MX
specification's bit-field definition and the sizes the Edge0 page prints."""
import json
import math
import os

import numpy as np
import pytest

from oracle import formats
from workloads import experts as wx

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def _bf16_bits(v: float) -> int:
    b = np.array([v], dtype=np.float32).view(np.uint32)[0]
    assert b & 0xFFFF == 0, "value must be exact in bf16"
    return int(b >> 16)


def test_int4_known_nibbles():
    # byte 0xF0: element 0 (low nibble) = 0, element 1 (high nibble) = 15
    out, inn = 1, 64
    q = np.full(inn // 2, 0x00, dtype=np.uint8)
    q[0] = 0xF0
    q[1] = 0x21                      # element 2 -> 1, element 3 -> 2
    s = np.array([_bf16_bits(0.015625)], dtype=np.uint16)
    b = np.array([_bf16_bits(-0.0625)], dtype=np.uint16)
    w = formats.dequant_int4(q, s, b, out, inn)
    assert w[0, 0] == -0.0625
    assert w[0, 1] == 0.015625 * 15 - 0.0625
    assert w[0, 2] == 0.015625 * 1 - 0.0625
    assert w[0, 3] == 0.015625 * 2 - 0.0625
    assert np.all(w[0, 4:] == -0.0625)


def test_int4_group_boundary():
    # two groups along the input: columns 0..63 use (s0, b0), 64..127 use (s1, b1)
    out, inn = 2, 128
    q = np.full(out * inn // 2, 0x77, dtype=np.uint8)   # every nibble 7
    s = np.array([_bf16_bits(v) for v in (0.5, 0.25, 1.0, 2.0)], dtype=np.uint16)
    b = np.array([_bf16_bits(v) for v in (1.0, -1.0, 0.0, 3.0)], dtype=np.uint16)
    w = formats.dequant_int4(q, s, b, out, inn)
    assert np.all(w[0, :64] == 7 * 0.5 + 1.0) and np.all(w[0, 64:] == 7 * 0.25 - 1.0)
    assert np.all(w[1, :64] == 7.0) and np.all(w[1, 64:] == 17.0)


def _e2m1_from_bits(code: int) -> float:
    """OCP MX v1.0 e2m1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent 0 is subnormal."""
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return sign * mag


def test_e2m1_table_matches_bitfield_definition():
    for c in range(16):
        assert formats.E2M1[c] == _e2m1_from_bits(c)
    assert formats.E2M1[0x7] == 6.0 and formats.E2M1[0xF] == -6.0 and formats.E2M1[0x1] == 0.5


def test_mxfp4_known_codes_and_scale():
    out, inn = 1, 64
    q = np.zeros(inn // 2, dtype=np.uint8)
    q[0] = 0xF7                       # element 0 -> +6, element 1 -> -6
    q[16] = 0x31                      # element 32 -> 0.5, element 33 -> 1.5
    e = np.array([127, 120], dtype=np.uint8)   # block 0: x1, block 1: x2**-7
    w = formats.dequant_mxfp4(q, e, out, inn)
    assert w[0, 0] == 6.0 and w[0, 1] == -6.0
    assert w[0, 32] == 0.5 * 2.0 ** -7 and w[0, 33] == 1.5 * 2.0 ** -7
    assert np.count_nonzero(w) == 4


def test_expert_size_reproduces_edge0_numbers():
    g = GOLD["expert_sizes"]
    S = formats.blob_size(formats.INT4_G64, g["hidden"], g["inter"])
    assert S == 1_769_472
    assert round(S / 1e6, 2) == g["mb_per_expert"]
    assert round(S * g["experts_per_layer"] / 1e6) == g["mb_per_layer"]
    total = S * g["experts_per_layer"] * g["layers"]
    assert round(total / 2 ** 30, 1) == g["gib_routed"]
    assert round(total / 1e9) == g["gb_routed"]
    # a plausible slip (group of 32, or fp32 scales) breaks the printed sizes
    assert round(3 * 2048 * 512 * (0.5 + 4 / 32) / 1e6, 2) != g["mb_per_expert"]
    assert round(3 * 2048 * 512 * (0.5 + 8 / 64) / 1e6, 2) != g["mb_per_expert"]


def test_generated_blob_layout_is_parsed_consistently():
    H, I = 128, 64
    for wfmt in (formats.INT4_G64, formats.MXFP4):
        blob = wx.expert_blob(7, 3, wfmt, H, I)
        assert blob.size == formats.blob_size(wfmt, H, I) == wx.expert_bytes(wfmt, H, I)
        wg, wu, wd = formats.dequant_expert(blob, wfmt, H, I)
        assert wg.shape == (I, H) and wu.shape == (I, H) and wd.shape == (H, I)
        assert np.all(np.isfinite(wg)) and np.all(np.isfinite(wd))


def test_generated_int4_value_ranges():
    H, I = 256, 128
    blob = wx.expert_blob(1000, 0, formats.INT4_G64, H, I)
    ng = I * H // 64
    s = formats.bf16_to_float(blob[I * H // 2: I * H // 2 + 2 * ng].view(np.uint16))
    b = formats.bf16_to_float(blob[I * H // 2 + 2 * ng: I * H // 2 + 4 * ng].view(np.uint16))
    assert s.min() >= 0.0049 and s.max() <= 0.0201
    assert np.all(b <= 0) and np.all(b >= -8 * s - 1e-6)
    q = formats.unpack_nibbles(blob[: I * H // 2])
    counts = np.bincount(q, minlength=16)
    assert counts.min() > 0.8 * counts.mean()


def test_generated_mx_exponent_range():
    H, I = 256, 128
    blob = wx.expert_blob(4000, 5, formats.MXFP4, H, I)
    e = blob[I * H // 2: I * H // 2 + I * H // 32]
    assert set(np.unique(e).tolist()) == {118, 119, 120, 121}
