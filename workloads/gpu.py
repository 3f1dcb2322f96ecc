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


def make_pool(w: Workload, n_layers: int | None = None, device="cuda") -> torch.Tensor:
    """All experts of ``n_layers`` layers (default: every layer), [L * E * S] uint8."""
    L = w.n_layers if n_layers is None else n_layers
    S = expert_bytes(w.wfmt, w.hidden, w.inter)
    pool = torch.empty(L * w.n_experts * S, dtype=torch.uint8, device=device)
    fill_experts(pool, 0, L * w.n_experts, w.wfmt, w.hidden, w.inter, seed(w.cid, 0))
    return pool
