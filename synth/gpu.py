"""Fill device tensors with the synthetic values of synth/weights.py, on the GPU (bit-identical)."""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict

import numpy as np
import torch

from . import weights as sw
from .configs import RunCfg, tensor_shapes

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsynth.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with `python -m synth.build`")
        lib = C.CDLL(path)
        lib.synth_fill.restype = C.c_int
        lib.synth_fill.argtypes = [C.c_void_p, C.c_uint64, C.c_uint64, C.c_void_p, C.c_int, C.c_void_p]
        _LIB = lib
    return _LIB


_TABLES: Dict[tuple, torch.Tensor] = {}


def _table(std: float, offset: float, dtype: str, device) -> torch.Tensor:
    k = (std, offset, dtype, str(device))
    if k not in _TABLES:
        bits = sw.table_bits(std, offset, dtype)
        t = torch.from_numpy(bits.view(np.int16 if dtype == "bf16" else np.int32).copy())
        _TABLES[k] = t.to(device)
    return _TABLES[k]


def fill(t: torch.Tensor, name: str, kind: str, seed: int, std: float, dtype: str, gain_std: float = 0.0):
    """Fill a contiguous device tensor (bf16/fp32 storage, or fp32 gains) with its synthetic values."""
    assert t.is_contiguous() and t.is_cuda
    if kind == "g":
        if gain_std == 0.0:
            t.fill_(1.0)
            return
        s, off, dt = gain_std, 1.0, "fp32"
    else:
        s, off, dt = std, 0.0, dtype
    assert t.element_size() == (2 if dt == "bf16" else 4)
    tab = _table(s, off, dt, t.device)
    rc = _lib().synth_fill(t.data_ptr(), t.numel(), sw.tensor_key(name, seed), tab.data_ptr(), t.element_size(),
                           torch.cuda.current_stream(t.device).cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill failed ({rc})")


def model_weights(cfg: RunCfg, device="cuda", gain_std: float = 0.0) -> Dict[str, torch.Tensor]:
    """All logical tensors of a run on the device.  Projections in the model dtype; gains fp32."""
    out = {}
    wdt = torch.bfloat16 if cfg.target.dtype == "bf16" else torch.float32
    for name, shape, kind in tensor_shapes(cfg.target, cfg.drafter):
        t = torch.empty(shape, dtype=torch.float32 if kind == "g" else wdt, device=device)
        fill(t, name, kind, cfg.weight_seed, cfg.weight_std, cfg.target.dtype, gain_std)
        out[name] = t
    return out
