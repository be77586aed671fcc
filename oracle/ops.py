"""Elementary operations of the decoder, written out from their definitions.

Sources (cited by short key throughout the oracle):
  [P1] "DFlash2 用投机解码给 Qwen 提速" (bml.asia)
  [P2] "你的大模型为啥突然快了，下一代投机解码 DFlash 拆给你看" (xiaodao.ai)
  [P3] "无损加速是真的吗？Qwen3.8-27B-DFlash2如何保证输出与目标模型完全一致" (rytg.cn)

[P3] section "结构一览" says the drafter is a Qwen3-structured stack; the
target is the Qwen3-family model it serves.  The pages do not restate the
Qwen3 layer, so the plainest reading is taken: pre-norm RMSNorm, grouped-
query attention with per-head RMSNorm on q and k, rotate-half RoPE, a SwiGLU
feed-forward, no biases.

Pins: tests/test_oracle_ops.py checks rms_norm against
torch.nn.functional.rms_norm, attention against
torch.nn.functional.scaled_dot_product_attention with explicit boolean masks,
and rope against its two invariants (norm preservation; q.k depends only on
the position difference) and a hand-computed 2-D rotation.
"""
from __future__ import annotations

import numpy as np


def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gain over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gain


def rope_angles(pos: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """Angles pos * theta^(-2i/d) for i in [0, d/2): shape [..., d/2]."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / head_dim)
    return np.asarray(pos, dtype=np.float64)[..., None] * inv_freq


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE.  x: [..., n_heads, d]; pos broadcast over [...] (one position per row).

    Pairs (i, i + d/2) are rotated by angle pos * theta^(-2i/d).
    """
    d = x.shape[-1]
    half = d // 2
    ang = rope_angles(pos, d, theta)[..., None, :]  # [..., 1, d/2]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def linear(x: np.ndarray, w: np.ndarray, rowwise: bool = False) -> np.ndarray:
    """y = x W^T for W stored [out, in].  rowwise=True evaluates each row as its own
    vector-matrix product, so a row's result never depends on which other rows share the call."""
    if rowwise:
        return np.stack([w @ row for row in x]) if len(x) else np.zeros((0, w.shape[0]), dtype=x.dtype)
    return x @ w.T


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """Masked softmax attention for one query row.

    q: [hq, d]; k, v: [n, hkv, d]; allowed: [n] boolean (which keys this query sees).
    Query head h reads KV head h // (hq / hkv).  Scores are scaled by 1/sqrt(d),
    the softmax subtracts the row maximum.  Returns [hq, d].
    """
    hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    out = np.zeros((hq, d), dtype=np.result_type(q, k))
    idx = np.nonzero(allowed)[0]
    if len(idx) == 0:
        return out
    scale = 1.0 / np.sqrt(d)
    for h in range(hq):
        kh = k[idx, h // group, :]
        vh = v[idx, h // group, :]
        s = (kh @ q[h]) * scale
        s = s - s.max()
        e = np.exp(s)
        w = e / e.sum()
        out[h] = w @ vh
    return out
