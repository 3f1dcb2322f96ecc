"""Expert weight formats, decoded the plain way.

int4 affine group-64 [Edge0, section 2 "Quantization": expert weights are int4
affine with groups of 64; section 3.1 "Executor paths": each projection carries
its packed weights plus scales and biases].  A weight is w = s * q + b with the
unsigned nibble q in 0..15 and bf16 s, b shared by 64 consecutive input
elements of one output row.

MXFP4 (OCP Microscaling Formats v1.0): an e2m1 element (sign bit 3, two
exponent bits, one mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) times
an e8m0 block scale 2**(E - 127) shared by 32 consecutive input elements.

Canonical blob layout of one expert: for gate [I, H], up [I, H], down [H, I] in
that order, int4 stores (q uint8 [out, in/2], s bf16 [out, in/64],
b bf16 [out, in/64]) and MXFP4 stores (q uint8 [out, in/2], e uint8
[out, in/32]).  Element 2c is the low nibble of byte c.
"""
from __future__ import annotations

import numpy as np

INT4_G64 = 0
MXFP4 = 1

# OCP MX v1.0, e2m1: code -> value (bit 3 is the sign)
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                 -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def bf16_to_float(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values (bf16 is the top half of fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """uint8 [..., n] -> uint8 [..., 2n]; element 2c = low nibble of byte c."""
    lo = packed & np.uint8(0x0F)
    hi = packed >> np.uint8(4)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequant_int4(q_packed: np.ndarray, s_bits: np.ndarray, b_bits: np.ndarray,
                 out: int, inn: int) -> np.ndarray:
    """w[o, i] = s[o, i // 64] * q[o, i] + b[o, i // 64] in float64."""
    q = unpack_nibbles(q_packed.reshape(out, inn // 2)).astype(np.float64)
    s = np.repeat(bf16_to_float(s_bits.reshape(out, inn // 64)), 64, axis=1)
    b = np.repeat(bf16_to_float(b_bits.reshape(out, inn // 64)), 64, axis=1)
    return s * q + b


def dequant_mxfp4(q_packed: np.ndarray, e_bytes: np.ndarray, out: int, inn: int) -> np.ndarray:
    """w[o, i] = e2m1(code[o, i]) * 2**(e[o, i // 32] - 127) in float64."""
    codes = unpack_nibbles(q_packed.reshape(out, inn // 2))
    scale = np.ldexp(1.0, e_bytes.reshape(out, inn // 32).astype(np.int64) - 127)
    return E2M1[codes] * np.repeat(scale, 32, axis=1)


def blob_size(wfmt: int, H: int, I: int) -> int:
    per_elem = {INT4_G64: 0.5 + 4.0 / 64.0, MXFP4: 0.5 + 1.0 / 32.0}[wfmt]
    return int(round(3 * H * I * per_elem))


def dequant_expert(blob: np.ndarray, wfmt: int, H: int, I: int):
    """Parse one canonical expert blob; returns float64 (W_gate [I,H], W_up [I,H], W_down [H,I])."""
    blob = np.asarray(blob, dtype=np.uint8)
    assert blob.size == blob_size(wfmt, H, I), (blob.size, blob_size(wfmt, H, I))
    mats = []
    off = 0
    for out, inn in ((I, H), (I, H), (H, I)):
        nq = out * inn // 2
        q = blob[off:off + nq]
        off += nq
        if wfmt == INT4_G64:
            ng = out * inn // 64
            s = blob[off:off + 2 * ng].view(np.uint16)
            off += 2 * ng
            b = blob[off:off + 2 * ng].view(np.uint16)
            off += 2 * ng
            mats.append(dequant_int4(q, s, b, out, inn))
        elif wfmt == MXFP4:
            ne = out * inn // 32
            e = blob[off:off + ne]
            off += ne
            mats.append(dequant_mxfp4(q, e, out, inn))
        else:
            raise ValueError(wfmt)
    assert off == blob.size
    return tuple(mats)


# ---- MX activation quantisation (OCP Microscaling Formats v1.0) -------------
# An MX block is 32 consecutive elements sharing one e8m0 scale X = 2**e; each
# element is stored in a narrow format after division by X.  For FP8 E4M3 (one
# sign bit, four exponent bits with bias 7, three mantissa bits; largest normal
# 1.75 * 2**8 = 448, no infinities) the shared exponent is
# e = floor(log2(max |v|)) - 8 (8 = the format's largest power of two), kept in
# e8m0's range [-127, 127]; elements are rounded to nearest (ties to even) and
# values beyond 448 saturate to 448.  A block of zeros takes e = -127.  This
# build stores every zero element as +0 (code 0x00).

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of one FP8 E4M3 code (0x7F and 0xFF are NaN)."""
    s, e, m = code >> 7, (code >> 3) & 0xF, code & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def mx_shared_exponent(amax: np.ndarray) -> np.ndarray:
    """e = floor(log2(amax)) - 8 clamped to [-127, 127]; -127 for amax = 0."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))      # amax = f * 2**ex, f in [0.5, 1)
    e = (ex - 1) - 8
    return np.where(amax > 0, np.clip(e, -127, 127), -127).astype(np.int64)


def e4m3_round(v: np.ndarray) -> np.ndarray:
    """Round to the nearest E4M3 value (ties to even), saturating at +-448."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    step = np.ldexp(1.0, np.maximum(ex - 1, -6) - 3)     # subnormals share 2**-9
    q = np.round(a / step) * step                         # numpy rounds halves to even
    return np.where(v < 0, -q, q) + 0.0                   # -0 becomes +0


def e4m3_encode(q: np.ndarray) -> np.ndarray:
    """Codes of values already on the E4M3 grid (|q| <= 448); zero is 0x00."""
    q = np.asarray(q, dtype=np.float64)
    a = np.abs(q)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    E = ex - 1
    normal = a >= 2.0 ** -6
    m = np.where(normal, np.ldexp(a, -E) * 8 - 8, a / 2.0 ** -9)
    e = np.where(normal, E + 7, 0)
    code = (e.astype(np.int64) << 3) | m.astype(np.int64)
    code = np.where(q < 0, code | 0x80, code)
    return np.where(a == 0, 0, code).astype(np.uint8)


def mx_quantize(v: np.ndarray, block: int = 32):
    """MX FP8 E4M3 quantisation along the last axis: (codes uint8 [..., n],
    scale bytes uint8 [..., n / 32] holding e + 127)."""
    v = np.asarray(v, dtype=np.float64)
    blocks = v.reshape(v.shape[:-1] + (v.shape[-1] // block, block))
    e = mx_shared_exponent(np.abs(blocks).max(axis=-1))
    q = e4m3_round(np.ldexp(blocks, -e[..., None]))
    return e4m3_encode(q).reshape(v.shape), (e + 127).astype(np.uint8)


def mx_dequantize(codes: np.ndarray, scales: np.ndarray, block: int = 32) -> np.ndarray:
    """Values of MX FP8 E4M3 data: code value * 2**(scale byte - 127)."""
    table = np.array([e4m3_value(c) for c in range(256)])
    vals = table[np.asarray(codes)]
    e = np.asarray(scales).astype(np.int64) - 127
    return np.ldexp(vals, np.repeat(e, block, axis=-1))


def mx_round_trip(v: np.ndarray) -> np.ndarray:
    """The MX FP8 E4M3 value each element of v is stored as."""
    return mx_dequantize(*mx_quantize(v))
