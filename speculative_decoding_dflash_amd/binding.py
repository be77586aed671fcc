"""ctypes binding of libdflash (include/dflash.h): the same names, argument marshalling only.

Device buffers are torch tensors (plumbing: memory and streams); every step of the decoding path
runs in the library's HIP kernels.  Importing this module fails loudly if the library is missing.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdflash.so")

MAX_TAPS = 16
MAX_BATCH = 64
MAX_BLOCK = 16
MAX_TOPK = 256
F16_MIN_ROWS = 32  # DFLASH_F16_MIN_ROWS

OK, E_INVAL, E_NOMEM, E_DEVICE, E_STATE = 0, -1, -2, -3, -4
BF16, F32 = 0, 1


class DflashError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"dflash status {status}: {msg}")
        self.status = status


class ModelCfg(C.Structure):
    _fields_ = [("layers", C.c_int32), ("hidden", C.c_int32), ("q_heads", C.c_int32), ("kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("ffn", C.c_int32), ("vocab", C.c_int32), ("rope_theta", C.c_float),
                ("rms_eps", C.c_float), ("dtype", C.c_int32)]


class DrafterCfg(C.Structure):
    _fields_ = [("layers", C.c_int32), ("n_taps", C.c_int32), ("taps", C.c_int32 * MAX_TAPS),
                ("block_size", C.c_int32), ("mask_id", C.c_int32), ("window", C.c_int32),
                ("conv_kernel", C.c_int32), ("conv_group", C.c_int32), ("selector_top_k", C.c_int32),
                ("selector_rank", C.c_int32)]


class LayerWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "ffn_norm",
                                          "w_gate", "w_up", "w_down", "w_conv")]


class TargetWeights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("final_norm", C.c_void_p), ("lm_head", C.c_void_p),
                ("layers", C.POINTER(LayerWeights))]


class DrafterWeights(C.Structure):
    _fields_ = [("fc", C.c_void_p), ("hidden_norm", C.c_void_p), ("final_norm", C.c_void_p),
                ("layers", C.POINTER(LayerWeights)), ("sel_u", C.c_void_p), ("sel_v", C.c_void_p)]


class Sampling(C.Structure):
    _fields_ = [("temperature", C.c_float), ("top_k", C.c_int32), ("top_p", C.c_float), ("seed", C.c_uint64)]


class Capacity(C.Structure):
    _fields_ = [("max_slots", C.c_int32), ("max_rows", C.c_int32), ("page_tokens", C.c_int32),
                ("num_pages", C.c_int32), ("max_pages_per_seq", C.c_int32)]


def _load() -> C.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m speculative_decoding_dflash_amd.build` "
                          "(there is no fallback path)")
    lib = C.CDLL(LIB_PATH)
    P, I, S, V = C.POINTER, C.c_int32, C.c_size_t, C.c_void_p
    sig = {
        "dflash_kv_pool_bytes": (S, [P(ModelCfg), I, P(Capacity)]),
        "dflash_drafter_pool_bytes": (S, [P(ModelCfg), P(DrafterCfg), P(Capacity)]),
        "dflash_workspace_bytes": (S, [P(ModelCfg), P(DrafterCfg), P(Capacity)]),
        "dflash_create": (I, [P(ModelCfg), P(DrafterCfg), P(TargetWeights), P(DrafterWeights), P(Capacity), V, V, V, V,
                              P(V)]),
        "dflash_destroy": (I, [V]),
        "dflash_kv_alloc": (I, [V, I, I]),
        "dflash_kv_free": (I, [V, I]),
        "dflash_verify_block": (I, [V, V, I, P(I), V, I, I, I, V, V]),
        "dflash_accept_resample": (I, [V, V, I, P(I), V, V, I, P(Sampling), V, V, V, V]),
        "dflash_draft_block": (I, [V, V, I, P(I), V, V, V]),
        "dflash_draft_block_sampled": (I, [V, V, I, P(I), V, P(Sampling), V, V, V, V]),
        "dflash_accept_resample_q": (I, [V, V, I, P(I), V, V, I, P(Sampling), V, V, V, V, V, V]),
        "dflash_device_status": (I, [V, V]),
        "dflash_op_linear": (I, [V, I, I, I, I, V, V, V]),
        "dflash_op_linear_f16x": (I, [V, I, I, I, V, V, V, I, P(I)]),
        "dflash_selector_state": (I, [V, V, I, V, V, V]),
        "dflash_op_linear_sk_scratch_bytes": (S, [I]),
        "dflash_op_linear_sk": (I, [V, I, I, I, I, V, V, V, V, S]),
        "dflash_op_linear_sk_noalloc": (I, [V, I, I, I, I, V, V, V]),
        "dflash_profile": (I, [V, I]),
        "dflash_profile_replay": (I, [V, V, I, P(C.c_double), P(C.c_double), P(I)]),
        "dflash_last_error": (C.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


def _check(status: int):
    if status != OK:
        raise DflashError(status, lib.dflash_last_error().decode())


def _ptr(t) -> Optional[int]:
    """Device address of a torch tensor (None passes NULL)."""
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _slots(slots: Sequence[int]):
    arr = (C.c_int32 * len(slots))(*[int(s) for s in slots])
    return arr


def dflash_kv_pool_bytes(cfg: ModelCfg, layers: int, cap: Capacity) -> int:
    return lib.dflash_kv_pool_bytes(C.byref(cfg), layers, C.byref(cap))


def dflash_drafter_pool_bytes(cfg: ModelCfg, dcfg: DrafterCfg, cap: Capacity) -> int:
    return lib.dflash_drafter_pool_bytes(C.byref(cfg), C.byref(dcfg), C.byref(cap))


def dflash_workspace_bytes(cfg: ModelCfg, dcfg: DrafterCfg, cap: Capacity) -> int:
    return lib.dflash_workspace_bytes(C.byref(cfg), C.byref(dcfg), C.byref(cap))


def dflash_create(cfg: ModelCfg, dcfg: DrafterCfg, tw: TargetWeights, dw: DrafterWeights, cap: Capacity, target_kv,
                  drafter_kv, workspace, stream=None) -> int:
    out = C.c_void_p()
    _check(lib.dflash_create(C.byref(cfg), C.byref(dcfg), C.byref(tw), C.byref(dw), C.byref(cap), _ptr(target_kv),
                             _ptr(drafter_kv), _ptr(workspace), _stream(stream), C.byref(out)))
    return out.value


def dflash_destroy(ctx: int):
    _check(lib.dflash_destroy(ctx))


def dflash_kv_alloc(ctx: int, slot: int, n_tokens: int):
    _check(lib.dflash_kv_alloc(ctx, slot, n_tokens))


def dflash_kv_free(ctx: int, slot: int):
    _check(lib.dflash_kv_free(ctx, slot))


def dflash_verify_block(ctx: int, slots: Sequence[int], tokens, q_len: int, new_sequence: bool, n_logit_rows: int,
                        logits, feats, stream=None):
    _check(lib.dflash_verify_block(ctx, _stream(stream), len(slots), _slots(slots), _ptr(tokens), q_len,
                                   int(bool(new_sequence)), n_logit_rows, _ptr(logits), _ptr(feats)))


def dflash_accept_resample(ctx: int, slots: Sequence[int], logits, block, n_draft: int, sampling: Sequence[Sampling],
                           out, n_out, cand_ids=None, cand_p=None, stream=None):
    sp = (Sampling * len(slots))(*sampling)
    _check(lib.dflash_accept_resample(ctx, _stream(stream), len(slots), _slots(slots), _ptr(logits), _ptr(block),
                                      n_draft, sp, _ptr(out), _ptr(n_out), _ptr(cand_ids), _ptr(cand_p)))


def dflash_draft_block(ctx: int, slots: Sequence[int], feats, block, logits=None, stream=None):
    _check(lib.dflash_draft_block(ctx, _stream(stream), len(slots), _slots(slots), _ptr(feats), _ptr(block),
                                  _ptr(logits)))


def dflash_draft_block_sampled(ctx: int, slots: Sequence[int], feats, sampling: Sequence[Sampling], block, q_ids, q_p,
                               logits=None, stream=None):
    sp = (Sampling * len(slots))(*sampling)
    _check(lib.dflash_draft_block_sampled(ctx, _stream(stream), len(slots), _slots(slots), _ptr(feats), sp,
                                          _ptr(block), _ptr(q_ids), _ptr(q_p), _ptr(logits)))


def dflash_accept_resample_q(ctx: int, slots: Sequence[int], logits, block, n_draft: int, sampling: Sequence[Sampling],
                             q_ids, q_p, out, n_out, cand_ids=None, cand_p=None, stream=None):
    sp = (Sampling * len(slots))(*sampling)
    _check(lib.dflash_accept_resample_q(ctx, _stream(stream), len(slots), _slots(slots), _ptr(logits), _ptr(block),
                                        n_draft, sp, _ptr(q_ids), _ptr(q_p), _ptr(out), _ptr(n_out), _ptr(cand_ids),
                                        _ptr(cand_p)))


def dflash_op_linear(dtype: int, M: int, N: int, K: int, x, w, y, stream=None):
    _check(lib.dflash_op_linear(_stream(stream), dtype, M, N, K, _ptr(x), _ptr(w), _ptr(y)))


def dflash_op_linear_f16x(M: int, N: int, K: int, x, w, y, max_ranges: int = 1, stream=None) -> int:
    """x fp16 [M, K], w bf16 [N, K], y fp32 [max_ranges, M, N]; returns the K ranges written."""
    n = C.c_int32(1)
    _check(lib.dflash_op_linear_f16x(_stream(stream), M, N, K, _ptr(x), _ptr(w), _ptr(y), max_ranges, C.byref(n)))
    return n.value


def dflash_selector_state(ctx: int, batch: int, ids, logits, trans, stream=None):
    """The last draft's selector candidates [batch, B-1, K] (ids, logits) and transitions [batch, B-1, K, K]."""
    _check(lib.dflash_selector_state(ctx, _stream(stream), batch, _ptr(ids), _ptr(logits), _ptr(trans)))


def dflash_op_linear_sk_scratch_bytes(N: int) -> int:
    return lib.dflash_op_linear_sk_scratch_bytes(N)


def dflash_op_linear_sk(dtype: int, M: int, N: int, K: int, x, w, y, scratch, stream=None):
    _check(lib.dflash_op_linear_sk(_stream(stream), dtype, M, N, K, _ptr(x), _ptr(w), _ptr(y), _ptr(scratch),
                                   scratch.numel() * scratch.element_size()))


def dflash_op_linear_sk_noalloc(dtype: int, M: int, N: int, K: int, x, w, y, stream=None):
    _check(lib.dflash_op_linear_sk_noalloc(_stream(stream), dtype, M, N, K, _ptr(x), _ptr(w), _ptr(y)))


def dflash_profile(ctx: int, enable: bool):
    _check(lib.dflash_profile(ctx, int(bool(enable))))


def dflash_profile_replay(ctx: int, iters: int, stream=None):
    """Replay the recorded projection launches: (elapsed ms, weight bytes per pass, launches per pass)."""
    ms, by, n = C.c_double(), C.c_double(), C.c_int32()
    _check(lib.dflash_profile_replay(ctx, _stream(stream), iters, C.byref(ms), C.byref(by), C.byref(n)))
    return ms.value, by.value, n.value


def dflash_device_status(ctx: int, stream=None):
    _check(lib.dflash_device_status(ctx, _stream(stream)))


def dflash_last_error() -> str:
    return lib.dflash_last_error().decode()
