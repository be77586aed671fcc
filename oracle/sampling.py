"""Sampling distribution, counter-based uniforms, and the accept / resample rule (oracle).

Sources: see oracle/ops.py for the [P1]/[P2]/[P3] keys.

* Sampling parameters temperature 1.0, top-p 0.95, top-k 20: [P1] paragraph
  introducing the model-card table; [P3] section "实测数据".  The pages give
  only the values.  Reading: scale logits by 1/T, keep the top-k by (value
  descending, token id ascending), softmax over those k, keep the smallest
  sorted prefix whose running sum reaches top_p (the crossing token is kept,
  at least one token is kept), renormalise.  T = 0 means greedy: all mass on
  the argmax (lowest id on ties).  top_k <= 0 keeps every token; top_p >= 1
  disables the nucleus cut.  All of this runs in float32 with sums taken
  sequentially in sorted order, because the GPU takes the same decisions in
  float32.
* Accept / resample ([P1] pseudocode and the sentence on rejection sampling
  in its cost-model paragraph; [P3] sections "先说结论" and "投机解码如何白嫖
  速度"): drafts are checked in order; the first rejected position is
  resampled from the target's own distribution and the step ends.  For the
  output law to equal plain decoding (the losslessness the pages promise), a
  deterministic draft x must be accepted with probability p(x) and a rejected
  position must be drawn from p with x removed and renormalised
  (norm(max(0, p - delta_x))).  When every draft is accepted, one more token
  is drawn from the last verified row (the bonus token), so a step emits
  between 1 and B tokens.
* Uniforms: Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random
  numbers: as easy as 1, 2, 3", SC 2011), key (seed, 0), counter
  (t, request, stream, 0) where t is the absolute position of the token being
  decided.  u_acc = (word0 >> 40) * 2^-24 and u_smp = (word1 >> 40) * 2^-24,
  both exact in float32 and in [0, 1).

* Stochastic drafts (the general rejection-sampling rule behind [P1]'s
  cost-model sentence on rejection sampling; the deterministic rule above is
  its special case): a draft drawn from the drafter's own filtered
  distribution q is accepted with probability min(1, p(x)/q(x)), taken in
  float32 as u_acc * q(x) < p(x); a rejected position is drawn from
  max(0, p - q) renormalised, over p's candidates in their order.  Reading
  where the pages are silent: the draft for position t is drawn from q by
  inverse CDF with the uniform u_draft = top 24 bits of word 0 of Philox
  counter (t, request, 1, 0) (stream 1; the target's decisions use stream 0),
  and q uses the request's own temperature / top-k / top-p.  With q a point
  mass at the draft, decide_q takes exactly decide's decisions.

Pins: tests/test_oracle_sampling.py -- Philox against numpy.random.Philox;
the filter against a brute-force sort and scipy's softmax; the rule's
accept rate (binomial z-test) and resample law (chi-square) against the
closed forms; greedy and B = 1 special cases; for stochastic drafts the
closed-form law (output marginal p, acceptance sum_x min(p, q)), a
Monte-Carlo chi-square of the float32 rule, and bit-equality with decide
when q is a point mass.  tests/test_oracle_spec.py enumerates the whole
loop's law with stochastic drafts against plain decoding.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

M64 = (1 << 64) - 1
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B

F32 = np.float32


def philox4x64_10(ctr: Sequence[int], key: Sequence[int]) -> Tuple[int, int, int, int]:
    """Ten rounds of Philox4x64 on a 4-word counter with a 2-word key (pure-integer arithmetic)."""
    c0, c1, c2, c3 = (int(v) & M64 for v in ctr)
    k0, k1 = (int(v) & M64 for v in key)
    for r in range(10):
        if r:
            k0 = (k0 + PHILOX_W0) & M64
            k1 = (k1 + PHILOX_W1) & M64
        p0 = PHILOX_M0 * c0
        p1 = PHILOX_M1 * c2
        hi0, lo0 = p0 >> 64, p0 & M64
        hi1, lo1 = p1 >> 64, p1 & M64
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def uniforms(seed: int, t: int, request: int, stream: int = 0) -> Tuple[np.float32, np.float32]:
    """(u_acc, u_smp) for the token at absolute position t of a request."""
    w = philox4x64_10((t, request, stream, 0), (seed, 0))
    return F32((w[0] >> 40) * 2.0 ** -24), F32((w[1] >> 40) * 2.0 ** -24)


def seq_sum(v: np.ndarray) -> np.float32:
    """Left-to-right float32 sum."""
    acc = F32(0.0)
    for x in np.asarray(v, dtype=np.float32):
        acc = F32(acc + x)
    return acc


def sample_dist(z: np.ndarray, temperature: float, top_k: int, top_p: float) -> Tuple[np.ndarray, np.ndarray]:
    """Candidate ids (sorted by scaled logit desc, id asc) and their float32 probabilities.

    Returns the kept candidates only; every other token has probability 0.
    """
    z = np.asarray(z, dtype=np.float32)
    vocab = z.shape[0]
    if temperature <= 0.0:
        best = int(np.argmax(z))  # first maximum = lowest id
        return np.array([best], dtype=np.int64), np.array([1.0], dtype=np.float32)
    s = z / F32(temperature)
    order = np.lexsort((np.arange(vocab), -s))  # primary: s descending; secondary: id ascending
    k = vocab if top_k <= 0 else min(top_k, vocab)
    ids = order[:k]
    e = np.exp(s[ids] - s[ids[0]]).astype(np.float32)
    q = (e / seq_sum(e)).astype(np.float32)
    keep = k
    if top_p < 1.0:
        acc = F32(0.0)
        for j in range(k):
            acc = F32(acc + q[j])
            if acc >= F32(top_p):
                keep = j + 1
                break
    kept_sum = seq_sum(q[:keep])
    p = (q[:keep] / kept_sum).astype(np.float32)
    return ids[:keep].astype(np.int64), p


def prob_of(ids: np.ndarray, p: np.ndarray, tok: int) -> np.float32:
    hit = np.nonzero(ids == tok)[0]
    return p[hit[0]] if len(hit) else F32(0.0)


def inverse_cdf(ids: np.ndarray, p: np.ndarray, u: np.float32, exclude: Optional[int]) -> int:
    """Draw from p (optionally with one token removed and the rest renormalised) with one uniform.

    S = sequential sum of the remaining probabilities, thr = u * S; the first
    remaining token whose running sum exceeds thr is drawn.  If rounding lets
    thr reach the total, the last remaining token with p > 0 is drawn.
    """
    keep = [j for j in range(len(ids)) if exclude is None or ids[j] != exclude]
    total = F32(0.0)
    for j in keep:
        total = F32(total + p[j])
    thr = F32(F32(u) * total)
    acc = F32(0.0)
    for j in keep:
        acc = F32(acc + p[j])
        if thr < acc:
            return int(ids[j])
    last = [j for j in keep if p[j] > 0]
    return int(ids[last[-1]])


def decide(rows: List[Tuple[np.ndarray, np.ndarray]], drafts: Sequence[int], n: int, seed: int,
           request: int) -> List[int]:
    """Accept / resample one verified block.

    rows[r] is the candidate distribution predicting position n + r + 1
    (r = 0 .. len(drafts)); drafts[i-1] is the draft for position n + i.
    Returns the emitted tokens (1 .. len(drafts)+1 of them).
    """
    out: List[int] = []
    for i, d in enumerate(drafts, start=1):
        ids, p = rows[i - 1]
        u_acc, u_smp = uniforms(seed, n + i, request)
        if u_acc < prob_of(ids, p, d):
            out.append(int(d))
            continue
        out.append(inverse_cdf(ids, p, u_smp, exclude=int(d)))
        return out
    ids, p = rows[len(drafts)]
    _, u_smp = uniforms(seed, n + len(drafts) + 1, request)
    out.append(inverse_cdf(ids, p, u_smp, exclude=None))
    return out


def sample_draft(ids: np.ndarray, q: np.ndarray, seed: int, t: int, request: int) -> int:
    """The draft for position t drawn from q (candidates ids, q) with u_draft of Philox stream 1."""
    u, _ = uniforms(seed, t, request, stream=1)
    return inverse_cdf(ids, q, u, exclude=None)


def residual(ids: np.ndarray, p: np.ndarray, qids: np.ndarray, q: np.ndarray) -> np.ndarray:
    """max(0, p - q) on p's candidates (float32, in p's candidate order)."""
    r = np.zeros(len(ids), dtype=np.float32)
    for j, y in enumerate(ids):
        d = F32(F32(p[j]) - prob_of(qids, q, int(y)))
        r[j] = d if d > F32(0.0) else F32(0.0)
    return r


def decide_q(rows: List[Tuple[np.ndarray, np.ndarray]], qrows: List[Tuple[np.ndarray, np.ndarray]],
             drafts: Sequence[int], n: int, seed: int, request: int) -> List[int]:
    """Accept / resample one verified block whose drafts were drawn from qrows[i-1] (float32 rule).

    Draft d_i is accepted iff u_acc * q(d_i) < p(d_i); at the first rejection the token is drawn by
    inverse CDF (u_smp) from max(0, p - q) over p's candidates, or from p itself should that residual
    vanish; after all accepts the bonus is drawn from the last row, as in ``decide``.
    """
    out: List[int] = []
    for i, d in enumerate(drafts, start=1):
        ids, p = rows[i - 1]
        qids, q = qrows[i - 1]
        u_acc, u_smp = uniforms(seed, n + i, request)
        if F32(u_acc * prob_of(qids, q, d)) < prob_of(ids, p, d):
            out.append(int(d))
            continue
        r = residual(ids, p, qids, q)
        out.append(inverse_cdf(ids, r, u_smp, exclude=None) if seq_sum(r) > F32(0.0)
                   else inverse_cdf(ids, p, u_smp, exclude=None))
        return out
    ids, p = rows[len(drafts)]
    _, u_smp = uniforms(seed, n + len(drafts) + 1, request)
    out.append(inverse_cdf(ids, p, u_smp, exclude=None))
    return out


def decide_q_law(rows: List[Tuple[np.ndarray, np.ndarray]], qrows: List[Tuple[np.ndarray, np.ndarray]],
                 drafts: Sequence[int]) -> List[Tuple[List[int], float]]:
    """Exact law (float64) of ``decide_q``'s output for fixed drafts: accept d_i with probability
    min(1, p(d_i) / q(d_i)); on rejection emit y with probability max(0, p(y) - q(y)) / sum of those."""
    out: List[Tuple[List[int], float]] = []
    acc = 1.0
    prefix: List[int] = []
    for i, d in enumerate(drafts, start=1):
        ids, p = rows[i - 1]
        qids, q = qrows[i - 1]
        p = np.asarray(p, dtype=np.float64)
        q = np.asarray(q, dtype=np.float64)
        pd = float(p[ids == d].sum())
        qd = float(q[qids == d].sum())
        a = 1.0 if qd <= pd else pd / qd
        if a < 1.0:
            r = np.array([max(0.0, float(py) - float(q[qids == y].sum())) for y, py in zip(ids, p)])
            tot = r.sum()
            for y, ry in zip(ids, r):
                if ry > 0:
                    out.append((prefix + [int(y)], acc * (1.0 - a) * ry / tot))
        acc *= a
        if acc == 0.0:
            return out
        prefix = prefix + [int(d)]
    ids, p = rows[len(drafts)]
    for y, py in zip(ids, np.asarray(p, dtype=np.float64)):
        if py > 0:
            out.append((prefix + [int(y)], acc * py))
    return out


def decide_law(rows: List[Tuple[np.ndarray, np.ndarray]], drafts: Sequence[int]) -> List[Tuple[List[int], float]]:
    """The exact law of ``decide``'s output (float64), for exact enumeration.

    Accept draft i with probability p_{i-1}(d_i); on rejection emit y != d_i
    with probability p_{i-1}(y) / (1 - p_{i-1}(d_i)); after all accepts emit
    the bonus y with probability p_last(y).
    """
    out: List[Tuple[List[int], float]] = []
    acc = 1.0
    prefix: List[int] = []
    for i, d in enumerate(drafts, start=1):
        ids, p = rows[i - 1]
        p = np.asarray(p, dtype=np.float64)
        pd = float(p[ids == d].sum())
        if pd < 1.0:
            rest = 1.0 - pd
            for y, py in zip(ids, p):
                if y != d and py > 0:
                    out.append((prefix + [int(y)], acc * rest * (py / rest)))
        acc *= pd
        if acc == 0.0:
            return out
        prefix = prefix + [int(d)]
    ids, p = rows[len(drafts)]
    for y, py in zip(ids, np.asarray(p, dtype=np.float64)):
        if py > 0:
            out.append((prefix + [int(y)], acc * py))
    return out


def sample_dist64(z: np.ndarray, temperature: float, top_k: int, top_p: float) -> Tuple[np.ndarray, np.ndarray]:
    """float64 version of sample_dist for exact law enumeration (same ordering rules)."""
    z = np.asarray(z, dtype=np.float64)
    vocab = z.shape[0]
    if temperature <= 0.0:
        return np.array([int(np.argmax(z))]), np.array([1.0])
    s = z / temperature
    order = np.lexsort((np.arange(vocab), -s))
    k = vocab if top_k <= 0 else min(top_k, vocab)
    ids = order[:k]
    e = np.exp(s[ids] - s[ids[0]])
    q = e / e.sum()
    keep = k
    if top_p < 1.0:
        c = np.cumsum(q)
        keep = int(np.nonzero(c >= top_p)[0][0]) + 1 if (c >= top_p).any() else k
    return ids[:keep].astype(np.int64), q[:keep] / q[:keep].sum()
