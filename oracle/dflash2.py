"""DFlash2 drafter variants: the 2-tap grouped dynamic convolution and the top-k / low-rank path selector
(oracle).  Test infrastructure: only tests, the smoke entry point and the benchmark's CPU baseline use it.

Source: [P3] section "DFlash 2 的三个设计" names three design points of the DFlash 2 drafter with their
configuration values only: block diffusion (the block drafter of oracle/model.py), a lightweight
selector that keeps 16 candidates per block position and, with a rank-256 selector, traces one globally
coherent path through them to hand to verification ("selector_top_k 16", "selector_rank 256"), and a
2-tap dynamic convolution in the backbone that steadies information flow inside the block
("conv_kernel_size 2", "conv_group_size 16").  The page gives no formulas; the definitions below are the
plainest readings that fit those names and values:

Dynamic convolution, in every drafter layer, on the attention input x = RMSNorm(h) * g (rows = the B
block positions of one request, in order):
    u_i      = W_conv x_i                                   (W_conv: [Kc * G, H], G = H / group)
    a_i[g,:] = softmax_t(u_i[g * Kc + t], t < Kc)           (one tap set per group of `group` channels)
    y_i[c]   = sum_{t < Kc, i - t >= 0} a_i[c // group, t] * x_{i-t}[c]
i.e. a causal convolution along the block whose Kc taps are computed from the current position
("dynamic") and shared by the channels of a group; positions before the block's first contribute zero.
The layer's q, k and v are projected from y instead of x.

Selector, after the drafter's LM head (z_i: logits of draft position i = 1 .. B-1):
    candidates c_i[0 .. K-1]: the K largest z_i, ordered by (logit desc, token id asc)
    phi(t) = U E[t], psi(t) = V E[t]   (U, V: [r, H] rank-r factors; E: the shared embedding table)
    T(a -> b) = phi(a) . psi(b) / sqrt(r)
    path score  S(k_1 .. k_{B-1}) = sum_i z_i[c_i[k_i]] + T(t_{i-1} -> t_i),  t_0 = anchor, t_i = c_i[k_i]
The drafts are the highest-scoring path, found by Viterbi: d_1(k) = z_1[k] + T(anchor -> c_1[k]);
d_i(k) = z_i[k] + max_k' (d_{i-1}(k') + T(c_{i-1}[k'] -> c_i[k])); the last position takes its best k
and every step back the predecessor that attained the max, the lowest index among equal values (the
reverse-lexicographically smallest optimal path).  Replacing argmax drafting by any rule keeps the
output law (the verification decides), so the selector changes only the acceptance length.

Precision: viterbi() runs in the dtype of its inputs with a fixed order of operations -- in float32,
(d + T) for every predecessor, the max, then + z -- the order the device follows, so that both take the
same decisions from the same float32 inputs.  Pins: tests/test_oracle_dflash2.py (brute force over all
paths, closed forms of the convolution, reduction to argmax drafting when the transitions vanish).
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np


def dyn_conv(x: np.ndarray, w_conv: np.ndarray, taps: int, group: int) -> np.ndarray:
    """Causal grouped dynamic convolution of the block rows x [B, H] (definition in the module doc)."""
    B, H = x.shape
    G = H // group
    u = (x @ w_conv.T).reshape(B, G, taps)
    u = u - u.max(axis=-1, keepdims=True)
    e = np.exp(u)
    a = e / e.sum(axis=-1, keepdims=True)  # [B, G, taps]
    y = np.zeros_like(x)
    for i in range(B):
        for t in range(taps):
            if i - t < 0:
                continue
            y[i] += np.repeat(a[i, :, t], group) * x[i - t]
    return y


def top_candidates(z: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """The k largest entries of z ordered by (value desc, index asc): (ids, values)."""
    order = np.lexsort((np.arange(len(z)), -z.astype(np.float64)))[:k]
    return order.astype(np.int64), z[order]


def transitions(embed: np.ndarray, sel_u: np.ndarray, sel_v: np.ndarray, src: Sequence[int],
                dst: Sequence[int]) -> np.ndarray:
    """T[a, b] = phi(src[a]) . psi(dst[b]) / sqrt(r) in float64."""
    r = sel_u.shape[0]
    phi = embed[np.asarray(src)].astype(np.float64) @ sel_u.T.astype(np.float64)
    psi = embed[np.asarray(dst)].astype(np.float64) @ sel_v.T.astype(np.float64)
    return phi @ psi.T / np.sqrt(r)


def viterbi(z: np.ndarray, trans: List[np.ndarray]) -> List[int]:
    """Best path through candidate scores z [n, K] with transitions trans[0] [1, K] (anchor -> row 0) and
    trans[i] [K, K] (row i-1 -> row i); returns the candidate index of every row.  Runs in z's dtype."""
    n, K = z.shape
    dt = z.dtype
    delta = (z[0] + trans[0][0].astype(dt)).astype(dt)
    back = np.zeros((n, K), dtype=np.int64)
    for i in range(1, n):
        new = np.empty(K, dtype=dt)
        for k in range(K):
            s = (delta + trans[i][:, k].astype(dt)).astype(dt)  # every predecessor
            j = int(np.argmax(s))  # first maximum: the lowest index among equal values
            back[i, k] = j
            new[k] = dt.type(s[j] + z[i, k])
        delta = new
    path = [int(np.argmax(delta))]
    for i in range(n - 1, 0, -1):
        path.append(int(back[i, path[-1]]))
    return path[::-1]


def select(logits: np.ndarray, anchor: int, embed: np.ndarray, sel_u: np.ndarray, sel_v: np.ndarray,
           k: int) -> List[int]:
    """Drafts of one block from the drafter's logits [B-1, V] (float64 throughout)."""
    cand = [top_candidates(row, k) for row in logits]
    ids = [c[0] for c in cand]
    z = np.stack([c[1] for c in cand]).astype(np.float64)
    trans = [transitions(embed, sel_u, sel_v, [anchor], ids[0])]
    for i in range(1, len(ids)):
        trans.append(transitions(embed, sel_u, sel_v, ids[i - 1], ids[i]))
    path = viterbi(z, trans)
    return [int(ids[i][path[i]]) for i in range(len(ids))]
