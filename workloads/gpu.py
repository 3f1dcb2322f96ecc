"""Device-side producer of synthetic expert pools (``libsynth355.so``).

The bytes equal ``workloads.experts.expert_blob`` for every expert; a test
checks that on sampled experts.  Input generation only.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .configs import Workload, seed
from .experts import expert_bytes

HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def _load():
    global _lib
    if _lib is None:
        path = os.path.join(HERE, "libsynth355.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} missing; run `python -m workloads.build`")
        _lib = ctypes.CDLL(path)
        _lib.synth_fill_experts.restype = ctypes.c_int
        _lib.synth_fill_experts.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_uint64, ctypes.c_void_p]
    return _lib


def fill_experts(dst: torch.Tensor, g0: int, count: int, wfmt: int, H: int, I: int,
                 seed_value: int) -> None:
    S = expert_bytes(wfmt, H, I)
    assert dst.dtype == torch.uint8 and dst.is_cuda and dst.numel() >= count * S
    st = torch.cuda.current_stream().cuda_stream
    rc = _load().synth_fill_experts(dst.data_ptr(), g0, count, wfmt, H, I, seed_value,
                                    ctypes.c_void_p(st))
    if rc != 0:
        raise RuntimeError(f"synth_fill_experts failed: hip error {rc}")


def make_pool(w: Workload, n_layers: int | None = None, device="cuda", pack=None) -> torch.Tensor:
    """All experts of ``n_layers`` layers (default: every layer), [L * E * S] uint8.

    The bytes are generated in the canonical layout; with ``pack(src, dst, n)``
    (the caller's layout conversion) each layer is generated into a scratch
    buffer and converted into the pool.
    """
    L = w.n_layers if n_layers is None else n_layers
    E = w.n_experts
    S = expert_bytes(w.wfmt, w.hidden, w.inter)
    pool = torch.empty(L * E * S, dtype=torch.uint8, device=device)
    if pack is None:
        fill_experts(pool, 0, L * E, w.wfmt, w.hidden, w.inter, seed(w.cid, 0))
        return pool
    scratch = torch.empty(E * S, dtype=torch.uint8, device=device)
    for l in range(L):
        fill_experts(scratch, l * E, E, w.wfmt, w.hidden, w.inter, seed(w.cid, 0))
        pack(scratch, pool[l * E * S:(l + 1) * E * S], E)
    del scratch
    return pool


def make_experts(w: Workload, g0: int, count: int, seed_value: int, pack=None,
                 device="cuda") -> torch.Tensor:
    """``count`` experts from global expert index ``g0``, canonical bytes converted
    by ``pack(src, dst, n)`` when given."""
    S = expert_bytes(w.wfmt, w.hidden, w.inter)
    raw = torch.empty(count * S, dtype=torch.uint8, device=device)
    fill_experts(raw, g0, count, w.wfmt, w.hidden, w.inter, seed_value)
    if pack is None:
        return raw
    out = torch.empty_like(raw)
    pack(raw, out, count)
    return out
