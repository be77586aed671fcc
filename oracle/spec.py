"""The speculative loop, the plain autoregressive loop, and their exact output laws (oracle).

Sources: see oracle/ops.py for the [P1]/[P2]/[P3] keys.

Loop ([P1] pseudocode and the paragraph after it; [P3] section
"投机解码如何白嫖速度"), with three readings where the printed skeleton is
generic or silent:
  * drafting is one parallel drafter forward over the block, not k serial
    drafter steps ([P1] paragraph after the pseudocode; [P2] "DFlash 的第一招");
  * a fully accepted block also emits the bonus token from the last verified
    row, so a step emits tau in 1 .. B tokens (tau is "tokens produced per
    verify step", [P3] section "实测数据");
  * output stops at exactly max_new tokens.
State of a sequence: n committed positions (target KV and injected drafter KV
valid for 0 .. n-1) and the anchor, the last emitted token, which sits at
position n.  One step verifies [anchor, d_1 .. d_{B-1}] at n .. n+B-1,
emits tau tokens, commits positions n .. n+tau-1 and injects their target
features into the drafter.  The prompt is handled as a step whose block is
the whole prompt with no drafts.  The first generated token counts toward
max_new.

With stochastic drafts (``stochastic=True``) each draft is drawn from the
drafter's own filtered distribution at its position (see sampling.decide_q);
the drafter's B-1 rows come from the same single forward, so the rows do not
depend on the drafts drawn before them.

Pins: greedy speculative output equals greedy autoregressive output token for
token ([P3] section "先说结论"); with B = 1 sampled speculative output equals
sampled autoregressive output bit for bit; exact enumeration of both output
laws on tiny models agrees to 1e-12 (the lossless claim of [P1] and [P3]),
with deterministic and with stochastic drafts; the planted-drafter mean
acceptance length matches its closed form.
"""
from __future__ import annotations

from collections import defaultdict
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

from .model import Drafter, KVCache, Target
from .sampling import decide, decide_law, decide_q, decide_q_law, sample_dist, sample_dist64, sample_draft


@dataclass
class Sampling:
    temperature: float = 1.0
    top_k: int = 20
    top_p: float = 0.95
    seed: int = 1

    @staticmethod
    def of(s) -> "Sampling":
        return Sampling(s.temperature, s.top_k, s.top_p, s.seed)


@dataclass
class SeqState:
    tcache: KVCache
    dcache: Optional[KVCache]
    n: int = 0
    anchor: int = -1
    out: List[int] = field(default_factory=list)
    taus: List[int] = field(default_factory=list)

    def copy(self) -> "SeqState":
        return SeqState(self.tcache.copy(), None if self.dcache is None else self.dcache.copy(), self.n,
                        self.anchor, list(self.out), list(self.taus))


class SpecDecoder:
    """Draft -> verify -> accept/resample, one sequence at a time."""

    def __init__(self, target: Target, drafter: Optional[Drafter], block_size: int, sampling: Sampling,
                 request: int = 0, stochastic: bool = False):
        self.target = target
        self.drafter = drafter
        self.B = block_size
        self.sp = sampling
        self.request = request
        self.stochastic = stochastic
        self.last_q = None  # the drafter's candidate distributions of the last stochastic block

    # -- one step, split so the law enumeration can branch between verify and commit
    def new_state(self) -> SeqState:
        return SeqState(self.target.new_cache(), None if self.drafter is None else self.drafter.new_cache())

    def block(self, st: SeqState, prompt: Optional[Sequence[int]],
              draft_fn: Optional[Callable[[SeqState], List[int]]] = None) -> Tuple[List[int], List[int]]:
        """Tokens to verify and the drafts among them."""
        if prompt is not None:
            return [int(t) for t in prompt], []
        if draft_fn is not None:
            drafts = [int(d) for d in draft_fn(st)]
        elif self.stochastic:
            self.last_q = self.draft_rows(st)
            drafts = [sample_draft(ids, q, self.sp.seed, st.n + i, self.request)
                      for i, (ids, q) in enumerate(self.last_q, start=1)]
        else:
            drafts = self.drafter.draft(st.dcache, st.anchor, st.n)
        return [st.anchor] + drafts, drafts

    def draft_rows(self, st: SeqState, exact: bool = False):
        """The drafter's filtered distributions q_1 .. q_{B-1} for the block at st.n."""
        return self.rows(self.drafter.draft_logits(st.dcache, st.anchor, st.n), exact)

    def verify(self, st: SeqState, tokens: List[int], drafts: List[int]):
        """Target forward over the block; logits of the last len(drafts)+1 rows and all features."""
        return self.target.forward(st.tcache, tokens, st.n, logit_rows=len(drafts) + 1)

    def rows(self, logits: np.ndarray, exact: bool = False):
        sp = self.sp
        if exact:
            return [sample_dist64(z, sp.temperature, sp.top_k, sp.top_p) for z in logits]
        return [sample_dist(z.astype(np.float32), sp.temperature, sp.top_k, sp.top_p) for z in logits]

    def commit(self, st: SeqState, tokens: List[int], drafts: List[int], emitted: List[int], feats: np.ndarray):
        start = st.n
        committed = len(tokens) - len(drafts) - 1 + len(emitted)
        if self.drafter is not None:
            self.drafter.inject(st.dcache, feats[:committed], start)
        st.n = start + committed
        st.anchor = emitted[-1]
        st.out.extend(emitted)
        st.taus.append(len(emitted))

    def step(self, st: SeqState, prompt: Optional[Sequence[int]] = None,
             draft_fn: Optional[Callable[[SeqState], List[int]]] = None) -> List[int]:
        tokens, drafts = self.block(st, prompt, draft_fn)
        logits, feats = self.verify(st, tokens, drafts)
        anchor_pos = st.n + len(tokens) - len(drafts) - 1
        if self.stochastic and drafts and draft_fn is None:
            emitted = decide_q(self.rows(logits), self.last_q, drafts, anchor_pos, self.sp.seed, self.request)
        else:
            emitted = decide(self.rows(logits), drafts, anchor_pos, self.sp.seed, self.request)
        self.commit(st, tokens, drafts, emitted, feats)
        return emitted

    def generate(self, prompt: Sequence[int], max_new: int,
                 draft_fn: Optional[Callable[[SeqState], List[int]]] = None) -> SeqState:
        st = self.new_state()
        self.step(st, prompt=prompt)
        while len(st.out) < max_new:
            self.step(st, draft_fn=draft_fn)
        st.out = st.out[:max_new]
        return st


def ar_generate(target: Target, prompt: Sequence[int], max_new: int, sampling: Sampling,
                request: int = 0) -> List[int]:
    """Plain decoding: one target forward per token, each token drawn with u_smp of its position."""
    cache = target.new_cache()
    logits, _ = target.forward(cache, prompt, 0, logit_rows=1)
    n = len(prompt)
    sp = sampling
    out: List[int] = []
    while True:
        row = sample_dist(logits[-1].astype(np.float32), sp.temperature, sp.top_k, sp.top_p)
        y = decide([row], [], n - 1, sp.seed, request)[0]
        out.append(y)
        if len(out) >= max_new:
            return out
        logits, _ = target.forward(cache, [y], n, logit_rows=1)
        n += 1


def ar_law(target: Target, prompt: Sequence[int], k: int, sampling: Sampling) -> Dict[Tuple[int, ...], float]:
    """Exact law of the first k generated tokens under plain decoding (float64).

    Every prefix is recomputed from scratch with a fresh cache, independently of
    the incremental cache logic used by the loops.
    """
    sp = sampling
    law: Dict[Tuple[int, ...], float] = {}

    def rec(prefix: Tuple[int, ...], prob: float):
        if len(prefix) == k:
            law[prefix] = law.get(prefix, 0.0) + prob
            return
        logits, _ = target.forward(target.new_cache(), list(prompt) + list(prefix), 0, logit_rows=1)
        ids, p = sample_dist64(logits[-1], sp.temperature, sp.top_k, sp.top_p)
        for y, py in zip(ids, p):
            if py > 0:
                rec(prefix + (int(y),), prob * float(py))

    rec((), 1.0)
    return law


def spec_law(dec: SpecDecoder, prompt: Sequence[int], k: int) -> Dict[Tuple[int, ...], float]:
    """Exact law of the first k tokens of the speculative loop (float64), branching on every
    accept / reject outcome with its probability and re-running the drafter per branch."""
    law: Dict[Tuple[int, ...], float] = defaultdict(float)

    def rec(st: SeqState, prob: float, prompt_block: Optional[Sequence[int]]):
        if len(st.out) >= k:
            law[tuple(st.out[:k])] += prob
            return
        if dec.stochastic and prompt_block is None:
            # branch on every draw of the drafts (each position from its own q) and then on every
            # accept / reject outcome
            qrows = dec.draft_rows(st, exact=True)
            combos = [([], 1.0)]
            for ids, q in qrows:
                combos = [(ds + [int(y)], pr * float(qy)) for ds, pr in combos for y, qy in zip(ids, q) if qy > 0]
            for drafts, pq in combos:
                s1 = st.copy()
                tokens = [s1.anchor] + drafts
                logits, feats = dec.verify(s1, tokens, drafts)
                for emitted, pe in decide_q_law(dec.rows(logits, exact=True), qrows, drafts):
                    if pe <= 0.0:
                        continue
                    s2 = s1.copy()
                    dec.commit(s2, tokens, drafts, emitted, feats)
                    rec(s2, prob * pq * pe, None)
            return
        tokens, drafts = dec.block(st, prompt_block)
        logits, feats = dec.verify(st, tokens, drafts)
        for emitted, pe in decide_law(dec.rows(logits, exact=True), drafts):
            if pe <= 0.0:
                continue
            s2 = st.copy()
            dec.commit(s2, tokens, drafts, emitted, feats)
            rec(s2, prob * pe, None)

    rec(dec.new_state(), 1.0, prompt)
    return dict(law)
