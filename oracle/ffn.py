"""Gathered quantised expert SwiGLU, the routing-weighted combine, and the
prefill permutation.

[Edge0, section 3.1 "Math contract"]: every executor path computes
down(silu(gate(x)) * up(x)) for each routed expert over its quantised weights,
checked element by element against a dequantised reference.  silu(z) =
z * sigmoid(z); no clamp, no bias vectors, no shared expert.

[FT-zh, Core method and Method steps]: the layer output of a token is the
routing-weighted sum of its experts' outputs; the GPU and CPU partial sums merge
exactly, so where an expert's bytes are read from (cache slot or pool) does not
change the result.  out[t] = sum_j w[t, j] * y[t, j], j ascending.

The prefill permutation groups the (token, slot) pairs by expert so each
expert runs once over its token bucket: a stable sort of the pairs p = t*k + j
by expert id, with offsets[e] the first position of expert e.
"""
from __future__ import annotations

import numpy as np

from .formats import MXFP4, dequant_expert, mx_round_trip


def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_expert(x: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """y = W_d (silu(W_g x) * (W_u x)) for each row of x [n, H]."""
    g = x @ wg.T
    u = x @ wu.T
    return (silu(g) * u) @ wd.T


def moe_layer(x: np.ndarray, ids: np.ndarray, w: np.ndarray, expert_blob, wfmt: int,
              H: int, I: int, dtype=np.float64, tokens=None) -> np.ndarray:
    """Layer output [len(tokens), H] for the selected tokens (all by default).

    ``expert_blob(e)`` returns the canonical S bytes of expert e.
    """
    x = np.asarray(x, dtype=dtype)
    ids = np.asarray(ids)
    w = np.asarray(w, dtype=dtype)
    T, k = ids.shape
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    row_of = {int(t): r for r, t in enumerate(tokens)}
    out = np.zeros((len(tokens), H), dtype=dtype)
    y = np.zeros((len(tokens), k, H), dtype=dtype)
    for e in sorted({int(v) for v in ids[tokens].ravel()}):
        wg, wu, wd = (m.astype(dtype) for m in dequant_expert(expert_blob(e), wfmt, H, I))
        pairs = [(t, j) for t in tokens for j in range(k) if ids[t, j] == e]
        rows = np.array([t for t, _ in pairs])
        ye = swiglu_expert(x[rows], wg, wu, wd)
        for (t, j), yrow in zip(pairs, ye):
            y[row_of[int(t)], j] = yrow
    return combine(y, w[tokens]).astype(dtype, copy=False)


def combine(y: np.ndarray, w: np.ndarray) -> np.ndarray:
    """out[t] = sum_j w[t, j] * y[t, j], slots j in ascending order.

    y [T, k, H] per-pair expert outputs, w [T, k] routing weights.
    """
    y = np.asarray(y)
    w = np.asarray(w)
    out = np.zeros((y.shape[0], y.shape[2]), dtype=np.result_type(y, w))
    for j in range(y.shape[1]):
        out += w[:, j][:, None] * y[:, j]
    return out


def moe_layer_mx8(x: np.ndarray, ids: np.ndarray, w: np.ndarray, expert_blob, H: int, I: int,
                  tokens=None) -> np.ndarray:
    """The layer over MXFP4 experts with MX FP8 E4M3 activations (OCP
    Microscaling v1.0), the operand pair of the native fp4 matrix-core path.

    Each token's x is quantised in blocks of 32 along H.  h = silu(g) * u is
    carried into the down projection as two MX terms, h1 = MX(h) and
    h2 = MX(h - h1), each quantised per routed pair in blocks of 32 along I:
    y = W_d (h1 + h2).  Float64 otherwise.
    """
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(ids)
    w = np.asarray(w, dtype=np.float64)
    T, k = ids.shape
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    row_of = {int(t): r for r, t in enumerate(tokens)}
    xq = mx_round_trip(x[tokens])
    y = np.zeros((len(tokens), k, H))
    for e in sorted({int(v) for v in ids[tokens].ravel()}):
        wg, wu, wd = dequant_expert(expert_blob(e), MXFP4, H, I)
        pairs = [(t, j) for t in tokens for j in range(k) if ids[t, j] == e]
        rows = np.array([row_of[int(t)] for t, _ in pairs])
        h = silu(xq[rows] @ wg.T) * (xq[rows] @ wu.T)
        h1 = mx_round_trip(h)
        h2 = mx_round_trip(h - h1)
        ye = (h1 + h2) @ wd.T
        for (t, j), yrow in zip(pairs, ye):
            y[row_of[int(t)], j] = yrow
    return combine(y, w[tokens])


def permute(ids: np.ndarray, n_experts: int):
    """perm int32 [T*k] (pair indices grouped by expert) and offsets int32 [E+1]."""
    flat = np.asarray(ids).ravel()
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    counts = np.bincount(flat, minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return perm, offsets
