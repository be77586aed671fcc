"""Pins of the DFlash2 drafter variants of the oracle (oracle/dflash2.py) against what their definitions
fix: the dynamic convolution's closed forms (uniform taps, saturated taps, group independence) and an
independent torch formulation; the selector's Viterbi against brute force over every path, its tie rule,
its reduction to argmax drafting when the transitions vanish, and a transition-forced path; the whole
speculative loop with both variants stays lossless (greedy speculative = greedy autoregressive)."""
import itertools

import numpy as np
import pytest
import torch

import synth
from oracle import dflash2
from oracle.model import Drafter, Target
from oracle.spec import Sampling, SpecDecoder, ar_generate
from synth import weights as sw


def test_dyn_conv_uniform_taps_average_neighbours():
    """W_conv = 0: both taps weigh 1/2, so row i is the mean of rows i and i-1 (row 0: half of itself)."""
    rng = np.random.default_rng(0)
    B, H, group = 5, 64, 16
    x = rng.standard_normal((B, H))
    y = dflash2.dyn_conv(x, np.zeros((2 * H // group, H)), 2, group)
    want = 0.5 * x
    want[1:] += 0.5 * x[:-1]
    assert np.allclose(y, want, atol=1e-15)


def test_dyn_conv_saturated_taps_are_identity():
    """Tap 0's logit far above tap 1's in every group: the convolution leaves the rows as they are (the
    drafter reduces to the plain block drafter)."""
    rng = np.random.default_rng(1)
    B, H, group = 4, 32, 16
    x = np.abs(rng.standard_normal((B, H))) + 1.0  # positive rows: u = W x has the sign of W's rows
    w = np.zeros((2 * H // group, H))
    w[0::2] = 100.0  # tap 0 of every group
    w[1::2] = -100.0
    assert np.allclose(dflash2.dyn_conv(x, w, 2, group), x, atol=1e-12)


def test_dyn_conv_groups_are_independent():
    """Changing the tap logits of group g changes only the channels of group g."""
    rng = np.random.default_rng(2)
    B, H, group = 6, 64, 16
    x = rng.standard_normal((B, H))
    w = rng.standard_normal((2 * H // group, H)) * 0.3
    w2 = w.copy()
    w2[2 * 1: 2 * 1 + 2] += rng.standard_normal((2, H))  # group 1's two taps
    a, b = dflash2.dyn_conv(x, w, 2, group), dflash2.dyn_conv(x, w2, 2, group)
    diff = np.abs(a - b).max(axis=0)
    assert (diff[group:2 * group] > 1e-6).all() and diff[:group].max() == 0 and diff[2 * group:].max() == 0


@pytest.mark.parametrize("taps", [1, 2, 3])
def test_dyn_conv_matches_torch_formulation(taps):
    """An independent formulation: softmax over tap logits grouped with torch, then a causal grouped
    convolution written as unfold over a zero-padded sequence."""
    rng = np.random.default_rng(3 + taps)
    B, H, group = 7, 48, 16
    G = H // group
    x = rng.standard_normal((B, H))
    w = rng.standard_normal((taps * G, H)) * 0.2
    tx = torch.from_numpy(x)
    a = torch.softmax((tx @ torch.from_numpy(w).T).view(B, G, taps), dim=-1)  # [B, G, taps]
    a = a.repeat_interleave(group, dim=1)                                       # [B, H, taps]
    pad = torch.cat([torch.zeros(taps - 1, H, dtype=tx.dtype), tx])            # [taps - 1 + B, H]
    win = pad.unfold(0, taps, 1)                                                # [B, H, taps]: rows i-taps+1 .. i
    y = (win.flip(-1) * a).sum(-1)                                              # tap t meets row i - t
    assert np.allclose(dflash2.dyn_conv(x, w, taps, group), y.numpy(), atol=1e-12)


def _brute(z, trans):
    """Best path by enumeration; among equal scores the reverse-lexicographically smallest."""
    n, K = z.shape
    best, arg = None, None
    for path in itertools.product(range(K), repeat=n):
        s = z[0, path[0]] + trans[0][0, path[0]]
        for i in range(1, n):
            s += z[i, path[i]] + trans[i][path[i - 1], path[i]]
        key = tuple(reversed(path))
        if best is None or s > best or (s == best and key < arg):
            best, arg = s, key
    return list(reversed(arg))


@pytest.mark.parametrize("n,K,seed", [(1, 5, 0), (3, 3, 1), (3, 4, 2), (4, 4, 3), (5, 3, 4)])
def test_viterbi_equals_brute_force(n, K, seed):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((n, K))
    trans = [rng.standard_normal((1, K))] + [rng.standard_normal((K, K)) for _ in range(n - 1)]
    assert dflash2.viterbi(z, trans) == _brute(z, trans)


@pytest.mark.parametrize("seed", range(6))
def test_viterbi_ties_take_the_lowest_indices(seed):
    """Integer-valued scores make exact ties common: the path is the reverse-lexicographically smallest
    of the optimal ones."""
    rng = np.random.default_rng(100 + seed)
    n, K = 4, 3
    z = rng.integers(0, 3, (n, K)).astype(np.float64)
    trans = [rng.integers(0, 2, (1, K)).astype(np.float64)] + [rng.integers(0, 2, (K, K)).astype(np.float64)
                                                               for _ in range(n - 1)]
    assert dflash2.viterbi(z, trans) == _brute(z, trans)


def test_viterbi_float32_keeps_its_order():
    """In float32 the rule adds the transition to the running score first, then the emission:
    (1 + 2^-24) + 2^-24 rounds to 1 (a tie with the other candidate, which the lower index wins), where
    1 + (2^-24 + 2^-24) would not; exact arithmetic prefers candidate 1."""
    e = 2.0 ** -24
    z = np.array([[1.0, 0.0], [0.0, e]])
    trans = [np.zeros((1, 2)), np.array([[0.0, e], [0.0, 0.0]])]
    assert dflash2.viterbi(z.astype(np.float32), [t.astype(np.float32) for t in trans]) == [0, 0]
    assert dflash2.viterbi(z, trans) == [0, 1]


def test_selector_without_transitions_is_argmax():
    """U = 0: every transition is 0 and the best path takes each row's best candidate, i.e. the argmax
    drafts of the pages' block drafter."""
    rng = np.random.default_rng(7)
    V, H, r, nd = 300, 32, 8, 5
    logits = rng.standard_normal((nd, V))
    embed = rng.standard_normal((V, H))
    d = dflash2.select(logits, 3, embed, np.zeros((r, H)), rng.standard_normal((r, H)), 16)
    assert d == [int(np.argmax(row)) for row in logits]


def test_selector_follows_strong_transitions():
    """With transitions far larger than the logit spread, the path follows the transition structure:
    here phi(a) . psi(b) rewards b = a + 1 among the candidates (rank 1 factors on a one-hot embedding)."""
    V, nd, K = 12, 3, 12
    embed = np.eye(V)
    u = np.zeros((2, V)); v = np.zeros((2, V))
    # phi(a) = (cos a t, sin a t), psi(b) = (cos (b - 1) t, sin (b - 1) t): the dot is maximal at b = a + 1
    th = 2 * np.pi / V
    u[0] = np.cos(th * np.arange(V)); u[1] = np.sin(th * np.arange(V))
    v[0] = np.cos(th * (np.arange(V) - 1)); v[1] = np.sin(th * (np.arange(V) - 1))
    u *= 100.0
    v *= 100.0
    rng = np.random.default_rng(8)
    logits = rng.standard_normal((nd, V)) * 0.01
    assert dflash2.select(logits, 4, embed, u, v, K) == [5, 6, 7]


def test_top_candidates_order():
    z = np.array([0.5, 2.0, 2.0, -1.0, 0.5, 3.0])
    ids, vals = dflash2.top_candidates(z, 4)
    assert ids.tolist() == [5, 1, 2, 0] and vals.tolist() == [3.0, 2.0, 2.0, 0.5]


def test_dflash2_drafter_loop_is_lossless():
    """The tiny model with both variants on: greedy speculative decoding emits the target's greedy
    stream token for token (the variants change only which drafts are proposed)."""
    cfg = synth.CONFIGS["tiny-dflash2"]
    W = sw.model_weights(cfg)
    t = Target(cfg.target, W, taps=cfg.drafter.taps)
    d = Drafter(cfg.target, cfg.drafter, W)
    prompt = sw.prompt_ids(cfg.target.vocab, cfg.drafter.mask_id, cfg.prompt_len, 0).tolist()
    g = Sampling(0.0, 0, 1.0, 1)
    ar = ar_generate(t, prompt, 24, g)
    st = SpecDecoder(t, d, cfg.drafter.block_size, g).generate(prompt, 24)
    assert st.out == ar
