"""Seeded synthetic expert weights in the canonical byte layout.

One expert is a contiguous blob.  int4 affine group-64 (the format the Edge0
page fixes in section 2 "Quantization" and section 3.1 "Executor paths": three
projections, each with packed weights, scales and biases):

    [gate_q, gate_s, gate_b, up_q, up_s, up_b, down_q, down_s, down_b]

MXFP4 (OCP Microscaling v1.0 e2m1 elements with an e8m0 scale per 32):

    [gate_q, gate_e, up_q, up_e, down_q, down_e]

``*_q`` is uint8 [out, in/2]; element 2c is the low nibble of byte c and 2c+1
the high nibble.  ``*_s`` / ``*_b`` are bf16 [out, in/64]; ``*_e`` is uint8
[out, in/32].  gate and up have out = I, in = H; down has out = H, in = I.

The bytes come from a counter-based generator, SplitMix64 (Steele, Lea and
Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014), so any
single expert can be regenerated on its own and a GPU kernel can produce a
whole pool with the same bytes.  Word ``j`` of region ``r`` of global expert
``g`` (= layer * E + expert) is

    mix64(base + (ctr + 1) * GAMMA),  ctr = g << 36 | r << 32 | j,
    base = mix64((seed + 1) * GAMMA)                      (all mod 2**64)

and the values are drawn from it as follows:

* packed nibbles / codes: the word's 8 bytes, little-endian, uniform 0..255;
* scale s (one word each): u = (word >> 40) * 2**-24, s = bf16(0.005 + 0.015 u)
  with fp32 multiply-then-add, each rounded to nearest even;
* bias b (one word each): u as above, b = bf16(fp32(-8 u) * fp32(s));
* e8m0 exponents: each byte of the word gives 118 + (byte & 3), scales
  2**-9 .. 2**-6.

This module holds no part of the layer's arithmetic.
"""
from __future__ import annotations

import numpy as np

from .configs import WFMT_INT4_G64, WFMT_MXFP4

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function on uint64 (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_base(seed: int) -> np.uint64:
    with np.errstate(over="ignore"):
        return mix64(np.uint64((seed + 1) & 0xFFFFFFFFFFFFFFFF) * GAMMA)[()]


def words(seed: int, g: int, region: int, n: int) -> np.ndarray:
    """n consecutive generator words of one region of one expert."""
    base = stream_base(seed)
    ctr = (np.uint64(g) << np.uint64(36)) | (np.uint64(region) << np.uint64(32))
    j = np.arange(n, dtype=np.uint64) + ctr + np.uint64(1)
    with np.errstate(over="ignore"):
        return mix64(base + j * GAMMA)


def f32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    b = np.asarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _uniform24(w: np.ndarray) -> np.ndarray:
    """Top 24 bits of each word as an exact float32 in [0, 1)."""
    return ((w >> np.uint64(40)).astype(np.float32)) * np.float32(2.0 ** -24)


def int4_scale_bias(seed: int, g: int, region_s: int, region_b: int, n: int):
    us = _uniform24(words(seed, g, region_s, n))
    s_f = np.float32(0.005) + (np.float32(0.015) * us).astype(np.float32)
    s_bits = f32_to_bf16_bits(s_f.astype(np.float32))
    ub = _uniform24(words(seed, g, region_b, n))
    v = (np.float32(-8.0) * ub).astype(np.float32)
    b_f = (v * bf16_bits_to_f32(s_bits)).astype(np.float32)
    return s_bits, f32_to_bf16_bits(b_f)


def packed_bytes(seed: int, g: int, region: int, nbytes: int) -> np.ndarray:
    assert nbytes % 8 == 0
    return words(seed, g, region, nbytes // 8).view(np.uint8).copy()


def mx_exponents(seed: int, g: int, region: int, n: int) -> np.ndarray:
    assert n % 8 == 0
    raw = words(seed, g, region, n // 8).view(np.uint8)
    return (np.uint8(118) + (raw & np.uint8(3))).astype(np.uint8)


def matrices(H: int, I: int):
    """(out, in) of gate, up, down."""
    return ((I, H), (I, H), (H, I))


def expert_bytes(wfmt: int, H: int, I: int) -> int:
    """Size S of one expert blob."""
    tot = 0
    for out, inn in matrices(H, I):
        if wfmt == WFMT_INT4_G64:
            tot += out * inn // 2 + 2 * (out * inn // 64) * 2
        elif wfmt == WFMT_MXFP4:
            tot += out * inn // 2 + out * inn // 32
        else:
            raise ValueError(wfmt)
    return tot


def expert_blob(seed: int, g: int, wfmt: int, H: int, I: int) -> np.ndarray:
    """The S bytes of global expert g (= layer * E + expert)."""
    parts = []
    for m, (out, inn) in enumerate(matrices(H, I)):
        if wfmt == WFMT_INT4_G64:
            ng = out * inn // 64
            parts.append(packed_bytes(seed, g, 3 * m + 0, out * inn // 2))
            s_bits, b_bits = int4_scale_bias(seed, g, 3 * m + 1, 3 * m + 2, ng)
            parts.append(s_bits.view(np.uint8))
            parts.append(b_bits.view(np.uint8))
        elif wfmt == WFMT_MXFP4:
            parts.append(packed_bytes(seed, g, 2 * m + 0, out * inn // 2))
            parts.append(mx_exponents(seed, g, 2 * m + 1, out * inn // 32))
        else:
            raise ValueError(wfmt)
    blob = np.concatenate(parts)
    assert blob.size == expert_bytes(wfmt, H, I)
    return blob


def layer_blob(seed: int, layer: int, n_experts: int, wfmt: int, H: int, I: int) -> np.ndarray:
    """All experts of one layer, expert-major [E * S] (the whole-layer buffer)."""
    return np.concatenate([expert_blob(seed, layer * n_experts + e, wfmt, H, I)
                           for e in range(n_experts)])
