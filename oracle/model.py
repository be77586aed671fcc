"""Target decoder and block-diffusion drafter with KV injection (oracle).

Sources: see oracle/ops.py for the [P1]/[P2]/[P3] keys.

Target ([P1] cost-model paragraph and pseudocode; [P2] section
"投机解码，让一个小弟先猜，大佬批量验"): a decoder whose KV cache holds every
committed position, so verifying a block of tokens is one forward over the
block that reads the cached prefix.  Keys are stored per absolute position;
rolling back rejected positions only moves the committed length, and the next
forward overwrites them.

Drafter ([P2] sections "DFlash 的第一招" and "DFlash 的第二招" and the SGLang
paragraph of "但研究跑通"; [P3] sections "DFlash 2 的三个设计" and
"结构一览"):
  * One forward fills a whole block [anchor, MASK x (B-1)] at positions
    n .. n+B-1; the output at mask position n+i is the draft for that
    position.  Block queries see every block key (bidirectional).
  * Target hidden states of committed positions are projected into every
    drafter layer's KV cache (KV injection) before drafting: concatenate the
    tapped layers' residual streams, apply the fc projection and an RMSNorm
    ("normalisation"), then each layer's own K/V projections, the per-head
    k-norm and RoPE ("positional encoding").  The cache holds only injected
    context positions; the block's own keys are written at n .. n+B-1, which
    the next injection overwrites.
  * Context keys are limited to a sliding window: query p sees context key
    k < n only when p - k < W (W = 0: no limit).
  * The drafter reuses the target's embedding table and LM head (the pages'
    1.92B parameter count only fits five 5120-wide layers plus fc when the
    vocabulary tables are shared).
  * Drafts are the argmax of float32 logits, ties to the lowest token id.

Readings where the pages are silent: taps are the residual stream after the
0-indexed target layer; the injected vector does not pass through a layer's
input RMSNorm (it is already normalised); the drafter's final RMSNorm is its
own.  Parity unpinned for this wiring (no reference implementation exists).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Sequence, Tuple

import numpy as np

from . import dflash2, ops


@dataclass
class Shape:
    layers: int
    hidden: int
    q_heads: int
    kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rope_theta: float
    rms_eps: float

    @staticmethod
    def of(cfg) -> "Shape":
        return Shape(cfg.layers, cfg.hidden, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.ffn, cfg.vocab,
                     cfg.rope_theta, cfg.rms_eps)


class KVCache:
    """Per-layer K and V indexed by absolute position; grows on demand."""

    def __init__(self, layers: int, kv_heads: int, head_dim: int, dtype, capacity: int = 64):
        self.k = [np.zeros((capacity, kv_heads, head_dim), dtype=dtype) for _ in range(layers)]
        self.v = [np.zeros((capacity, kv_heads, head_dim), dtype=dtype) for _ in range(layers)]

    def ensure(self, n: int):
        cap = self.k[0].shape[0]
        if n <= cap:
            return
        new = max(n, 2 * cap)
        for arrs in (self.k, self.v):
            for i, a in enumerate(arrs):
                b = np.zeros((new,) + a.shape[1:], dtype=a.dtype)
                b[:cap] = a
                arrs[i] = b

    def write(self, layer: int, pos: np.ndarray, k: np.ndarray, v: np.ndarray):
        self.ensure(int(pos.max()) + 1)
        self.k[layer][pos] = k
        self.v[layer][pos] = v

    def copy(self) -> "KVCache":
        c = KVCache.__new__(KVCache)
        c.k = [a.copy() for a in self.k]
        c.v = [a.copy() for a in self.v]
        return c


def _layer_qkv(w: Dict[str, np.ndarray], p: str, s: Shape, x: np.ndarray, pos: np.ndarray, rowwise: bool,
               conv: Tuple[int, int] = (0, 0)):
    """Pre-norm, q/k/v projections, per-head q/k RMSNorm and RoPE for rows x at positions pos.
    conv = (taps, group): the normed rows (one block, in order) first pass through the DFlash2 dynamic
    convolution (oracle/dflash2.py)."""
    xn = ops.rms_norm(x, w[p + "attn_norm"], s.rms_eps)
    if conv[0]:
        xn = dflash2.dyn_conv(xn, w[p + "w_conv"], conv[0], conv[1])
    q = ops.linear(xn, w[p + "wq"], rowwise).reshape(len(x), s.q_heads, s.head_dim)
    k = ops.linear(xn, w[p + "wk"], rowwise).reshape(len(x), s.kv_heads, s.head_dim)
    v = ops.linear(xn, w[p + "wv"], rowwise).reshape(len(x), s.kv_heads, s.head_dim)
    q = ops.rope(ops.rms_norm(q, w[p + "q_norm"], s.rms_eps), pos, s.rope_theta)
    k = ops.rope(ops.rms_norm(k, w[p + "k_norm"], s.rms_eps), pos, s.rope_theta)
    return q, k, v


def _layer_out_ffn(w: Dict[str, np.ndarray], p: str, s: Shape, x: np.ndarray, attn: np.ndarray, rowwise: bool):
    """Output projection + residual, then pre-norm SwiGLU feed-forward + residual."""
    x = x + ops.linear(attn.reshape(len(x), -1), w[p + "wo"], rowwise)
    xn = ops.rms_norm(x, w[p + "ffn_norm"], s.rms_eps)
    g = ops.linear(xn, w[p + "w_gate"], rowwise)
    u = ops.linear(xn, w[p + "w_up"], rowwise)
    return x + ops.linear(ops.silu(g) * u, w[p + "w_down"], rowwise)


class Target:
    """Qwen3-like decoder with a position-indexed KV cache."""

    def __init__(self, cfg, weights: Dict[str, np.ndarray], taps: Sequence[int] = (), dtype=np.float64,
                 rowwise: bool = False):
        self.s = Shape.of(cfg)
        self.w = {k: v.astype(dtype) for k, v in weights.items() if k.startswith("t.")}
        self.taps = tuple(taps)
        self.dtype = dtype
        self.rowwise = rowwise

    def new_cache(self) -> KVCache:
        return KVCache(self.s.layers, self.s.kv_heads, self.s.head_dim, self.dtype)

    def forward(self, cache: KVCache, tokens: Sequence[int], start: int,
                logit_rows: int = -1) -> Tuple[np.ndarray, np.ndarray]:
        """Run tokens at positions start .. start+q-1 over the cached prefix 0 .. start-1.

        Writes the block's K/V into the cache.  Query at position p sees keys 0 .. p.
        Returns (logits of the last ``logit_rows`` rows (all rows if -1), features
        [q, n_taps, hidden] = residual stream after each tapped layer).
        """
        s, w = self.s, self.w
        toks = np.asarray(tokens, dtype=np.int64)
        q_len = len(toks)
        pos = np.arange(start, start + q_len)
        x = w["t.embed"][toks].copy()
        feats = np.zeros((q_len, len(self.taps), s.hidden), dtype=self.dtype)
        for l in range(s.layers):
            p = f"t.L{l}."
            q, k, v = _layer_qkv(w, p, s, x, pos, self.rowwise)
            cache.write(l, pos, k, v)
            attn = np.stack([ops.attention(q[i], cache.k[l][:pos[i] + 1], cache.v[l][:pos[i] + 1],
                                           np.ones(pos[i] + 1, dtype=bool)) for i in range(q_len)])
            x = _layer_out_ffn(w, p, s, x, attn, self.rowwise)
            if l in self.taps:
                feats[:, self.taps.index(l)] = x
        rows = q_len if logit_rows < 0 else logit_rows
        xn = ops.rms_norm(x[q_len - rows:], w["t.final_norm"], s.rms_eps)
        return ops.linear(xn, w["t.lm_head"], self.rowwise), feats


class Drafter:
    """Block-diffusion drafter with per-layer KV injection of target features."""

    def __init__(self, tcfg, dcfg, weights: Dict[str, np.ndarray], dtype=np.float64, rowwise: bool = False):
        self.s = Shape.of(tcfg)
        self.d = dcfg
        self.w = {k: v.astype(dtype) for k, v in weights.items() if k.startswith("d.")}
        self.embed = weights["t.embed"].astype(dtype)
        self.lm_head = weights["t.lm_head"].astype(dtype)
        self.dtype = dtype
        self.rowwise = rowwise

    def new_cache(self) -> KVCache:
        return KVCache(self.d.layers, self.s.kv_heads, self.s.head_dim, self.dtype)

    def inject(self, cache: KVCache, feats: np.ndarray, start: int):
        """Project target features of positions start .. start+r-1 into every layer's cache.

        c = RMSNorm(W_fc [h_tap1; ...; h_tapm]);  K_j = RoPE(knorm_j(W_k^j c));  V_j = W_v^j c.
        """
        r = len(feats)
        if r == 0:
            return
        s, w = self.s, self.w
        pos = np.arange(start, start + r)
        c = ops.linear(feats.reshape(r, -1), w["d.fc"], self.rowwise)
        c = ops.rms_norm(c, w["d.hidden_norm"], s.rms_eps)
        for j in range(self.d.layers):
            p = f"d.L{j}."
            k = ops.linear(c, w[p + "wk"], self.rowwise).reshape(r, s.kv_heads, s.head_dim)
            v = ops.linear(c, w[p + "wv"], self.rowwise).reshape(r, s.kv_heads, s.head_dim)
            k = ops.rope(ops.rms_norm(k, w[p + "k_norm"], s.rms_eps), pos, s.rope_theta)
            cache.write(j, pos, k, v)

    def draft_logits(self, cache: KVCache, anchor: int, n: int) -> np.ndarray:
        """Logits [B-1, V] of the mask positions n+1 .. n+B-1 of block [anchor, MASK x (B-1)] at n .. n+B-1."""
        s, w, B, W = self.s, self.w, self.d.block_size, self.d.window
        toks = np.array([anchor] + [self.d.mask_id] * (B - 1), dtype=np.int64)
        pos = np.arange(n, n + B)
        x = self.embed[toks].copy()
        keys = np.arange(n + B)
        conv = (self.d.conv_kernel, self.d.conv_group)
        for j in range(self.d.layers):
            p = f"d.L{j}."
            q, k, v = _layer_qkv(w, p, s, x, pos, self.rowwise, conv)
            cache.write(j, pos, k, v)
            attn = []
            for i in range(B):
                ctx_ok = (keys < n) & ((W <= 0) | (pos[i] - keys < W))
                allowed = ctx_ok | (keys >= n)
                attn.append(ops.attention(q[i], cache.k[j][:n + B], cache.v[j][:n + B], allowed))
            x = _layer_out_ffn(w, p, s, x, np.stack(attn), self.rowwise)
        xn = ops.rms_norm(x[1:], w["d.final_norm"], s.rms_eps)
        return ops.linear(xn, self.lm_head, self.rowwise)

    def draft(self, cache: KVCache, anchor: int, n: int) -> List[int]:
        """Argmax drafts, or with the DFlash2 selector the best path through its candidates."""
        z = self.draft_logits(cache, anchor, n)
        if self.d.selector_top_k:
            return dflash2.select(z, anchor, self.embed, self.w["d.sel_u"], self.w["d.sel_v"], self.d.selector_top_k)
        z = z.astype(np.float32)
        return [int(np.argmax(row)) for row in z]
