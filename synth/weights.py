"""Seeded, counter-based synthetic weights and workloads.

This module only makes inputs.  It holds none of the decoding method's
arithmetic, so both the CPU oracle and the GPU path may use it.

Definition of every generated value (the CPU code below and the GPU fill
kernel in ``gen.hip`` implement the same definition and must agree bit for
bit):

* ``mix64(z)`` is the SplitMix64 finaliser (Steele, Lea and Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014):
  ``z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27; z *= 0x94D049BB133111EB;
  z ^= z >> 31`` with arithmetic mod 2**64.
* A tensor's key is ``mix64(fnv1a64(name) ^ (seed * GOLDEN))`` where GOLDEN is
  0x9E3779B97F4A7C15 and ``fnv1a64`` is the 64-bit FNV-1a hash of the UTF-8
  name.
* Element ``i`` of the row-major tensor takes the 64-bit word
  ``w = mix64(key + (i // 4 + 1) * GOLDEN)`` and the 16-bit lane
  ``u = (w >> (16 * (i % 4))) & 0xFFFF``.
* A projection element is ``table[u]`` with ``table[u] = round(std *
  Phi^-1((u + 0.5) / 65536))``: the normal quantile function evaluated on a
  65536-point grid, rounded to float32 and then (for bf16 models) to bfloat16
  with round-to-nearest-even.  The distribution is N(0, std) quantised to
  65536 equiprobable levels; it is truncated at about 4.3 std.
* An RMSNorm gain is 1.0 unless ``gain_std`` > 0, in which case it is
  ``1 + gain_std * Phi^-1(...)`` on the same grid (used by tests so that a
  dropped gain cannot go unnoticed).
"""
from __future__ import annotations

import statistics
from functools import lru_cache
from typing import Dict, Iterable, Optional, Sequence

import numpy as np

from .configs import DecoderCfg, DrafterCfg, RunCfg, tensor_shapes

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
MIX_M1 = 0xBF58476D1CE4E5B9
MIX_M2 = 0x94D049BB133111EB


def fnv1a64(name: str) -> int:
    h = 0xCBF29CE484222325
    for b in name.encode("utf-8"):
        h ^= b
        h = (h * 0x100000001B3) & MASK64
    return h


def mix64_int(z: int) -> int:
    z &= MASK64
    z ^= z >> 30
    z = (z * MIX_M1) & MASK64
    z ^= z >> 27
    z = (z * MIX_M2) & MASK64
    z ^= z >> 31
    return z


def mix64_np(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= np.uint64(MIX_M1)
        z ^= z >> np.uint64(27)
        z *= np.uint64(MIX_M2)
        z ^= z >> np.uint64(31)
    return z


def tensor_key(name: str, seed: int) -> int:
    return mix64_int(fnv1a64(name) ^ ((seed * GOLDEN) & MASK64))


def words(key: int, j: np.ndarray) -> np.ndarray:
    """64-bit words number j (0-based) of the stream with this key."""
    with np.errstate(over="ignore"):
        z = np.uint64(key) + (j.astype(np.uint64) + np.uint64(1)) * np.uint64(GOLDEN)
    return mix64_np(z)


def lanes16(key: int, start: int, count: int) -> np.ndarray:
    """16-bit uniforms for elements start .. start+count-1 of a tensor stream."""
    if count == 0:
        return np.zeros(0, dtype=np.uint16)
    j0, j1 = start // 4, (start + count - 1) // 4
    w = words(key, np.arange(j0, j1 + 1, dtype=np.uint64))
    lanes = np.stack([(w >> np.uint64(16 * s)) & np.uint64(0xFFFF) for s in range(4)], axis=1).reshape(-1)
    off = start - 4 * j0
    return lanes[off:off + count].astype(np.uint16)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@lru_cache(maxsize=None)
def _quantiles() -> np.ndarray:
    nd = statistics.NormalDist()
    return np.array([nd.inv_cdf((u + 0.5) / 65536.0) for u in range(65536)], dtype=np.float64)


@lru_cache(maxsize=None)
def value_table(std: float, offset: float, dtype: str) -> np.ndarray:
    """65536-entry lookup table: float32 values, already rounded to the storage dtype."""
    v = (offset + std * _quantiles()).astype(np.float32)
    if dtype == "bf16":
        v = bf16_bits_to_f32(f32_to_bf16_bits(v))
    return v


def table_bits(std: float, offset: float, dtype: str) -> np.ndarray:
    """The table as raw storage bits (uint16 for bf16, uint32 for fp32) for the GPU fill kernel."""
    t = value_table(std, offset, dtype)
    return f32_to_bf16_bits(t) if dtype == "bf16" else t.view(np.uint32).copy()


def tensor_elements(name: str, seed: int, std: float, offset: float, dtype: str, start: int,
                    count: int) -> np.ndarray:
    """float32 values (exactly representable in the storage dtype) of elements start..start+count-1."""
    return value_table(std, offset, dtype)[lanes16(tensor_key(name, seed), start, count)]


def tensor(name: str, shape: Sequence[int], kind: str, seed: int, std: float, dtype: str,
           gain_std: float = 0.0, rows: Optional[Iterable[int]] = None) -> np.ndarray:
    """A whole tensor (or selected rows of a 2-D tensor) as float32 values."""
    shape = tuple(shape)
    if kind == "g":
        if gain_std == 0.0:
            return np.ones(shape, dtype=np.float32)
        s, off = gain_std, 1.0
    else:
        s, off = std, 0.0
    if rows is None:
        n = int(np.prod(shape))
        return tensor_elements(name, seed, s, off, dtype, 0, n).reshape(shape)
    rows = list(rows)
    cols = shape[1]
    out = np.empty((len(rows), cols), dtype=np.float32)
    for i, r in enumerate(rows):
        out[i] = tensor_elements(name, seed, s, off, dtype, r * cols, cols)
    return out


def model_weights(cfg: RunCfg, gain_std: float = 0.0, names: Optional[Iterable[str]] = None) -> Dict[str, np.ndarray]:
    """All (or the named) logical tensors of a run's target + drafter, as float32 numpy arrays."""
    want = None if names is None else set(names)
    out = {}
    for name, shape, kind in tensor_shapes(cfg.target, cfg.drafter):
        if want is not None and name not in want:
            continue
        out[name] = tensor(name, shape, kind, cfg.weight_seed, cfg.weight_std, cfg.target.dtype, gain_std)
    return out


# ---------------------------------------------------------------- workloads

def _stream_words(tag: str, seed: int, idx: np.ndarray) -> np.ndarray:
    return words(tensor_key(tag, seed), idx)


def prompt_ids(vocab: int, mask_id: int, length: int, request: int, seed: int = 0) -> np.ndarray:
    """Prompt token ids, i.i.d. uniform over [0, vocab) without the mask id."""
    w = _stream_words(f"prompt/{request}", seed, np.arange(length, dtype=np.uint64))
    r = (w % np.uint64(vocab - 1)).astype(np.int64)
    r += (r >= mask_id).astype(np.int64)
    return r.astype(np.int32)


def prompt_lengths(lo: int, hi: int, n: int, seed: int = 0) -> np.ndarray:
    """Per-request prompt lengths, uniform over lo..hi inclusive."""
    w = _stream_words("prompt_len", seed, np.arange(n, dtype=np.uint64))
    return (lo + (w % np.uint64(hi - lo + 1)).astype(np.int64)).astype(np.int32)


def planted_drafts(greedy_stream: np.ndarray, start: int, n_draft: int, vocab: int, mask_id: int,
                   rate: float, request: int = 0, seed: int = 1,
                   force_reject_at: Optional[int] = None) -> np.ndarray:
    """A planted drafter: drafts for positions start+1 .. start+n_draft.

    ``greedy_stream[t]`` is the target's greedy token at absolute position t.
    Each draft equals that token unless it is corrupted: corruption happens
    independently per absolute position with probability ``rate`` (uniform
    from the counter-based stream ``plant/<request>``), and the replacement is
    uniform over the tokens other than the greedy one and the mask id.  With
    ``force_reject_at = j`` (1-based) drafts 1..j-1 are clean and draft j is
    always corrupted, so greedy verification accepts exactly j-1 drafts.
    """
    pos = np.arange(start + 1, start + 1 + n_draft, dtype=np.uint64)
    key = tensor_key(f"plant/{request}", seed)
    w1 = words(key, 2 * pos)
    w2 = words(key, 2 * pos + np.uint64(1))
    u = (w1 >> np.uint64(40)).astype(np.float64) * 2.0 ** -24
    corrupt = u < rate
    if force_reject_at is not None:
        corrupt = np.zeros(n_draft, dtype=bool)
        if force_reject_at <= n_draft:
            corrupt[force_reject_at - 1:] = True
    g = greedy_stream[start + 1:start + 1 + n_draft].astype(np.int64)
    out = g.copy()
    for i in np.nonzero(corrupt)[0]:
        excluded = sorted({int(g[i]), int(mask_id)})
        x = int(w2[i] % np.uint64(vocab - len(excluded)))
        for e in excluded:
            if x >= e:
                x += 1
        out[i] = x
    return out.astype(np.int32)
