"""Pins of the oracle's loops: greedy exactness, B = 1 reduction, exact law equality, KV rollback,
and the planted drafter's closed-form acceptance length."""
from dataclasses import replace

import numpy as np
import pytest
import scipy.stats

import synth
from oracle.model import Drafter, Target
from oracle.spec import Sampling, SpecDecoder, ar_generate, ar_law, spec_law
from synth import weights as sw


def tiny_models(rowwise=False):
    cfg = synth.TINY
    W = sw.model_weights(cfg, gain_std=0.1)
    tg = Target(cfg.target, W, taps=cfg.drafter.taps, rowwise=rowwise)
    dr = Drafter(cfg.target, cfg.drafter, W, rowwise=rowwise)
    prompt = sw.prompt_ids(cfg.target.vocab, cfg.drafter.mask_id, cfg.prompt_len, 0)
    return cfg, tg, dr, prompt


def micro_cfg(vocab=6, block=3, std=0.6, window=0):
    t = synth.DecoderCfg(layers=2, hidden=16, q_heads=2, kv_heads=1, head_dim=8, ffn=32, vocab=vocab,
                         rope_theta=1e4, dtype="fp32")
    d = synth.DrafterCfg(layers=1, taps=(0, 1), block_size=block, mask_id=vocab - 1, window=window)
    return synth.RunCfg(name="micro", target=t, drafter=d, prompt_len=2, gen_len=4, weight_std=std)


def micro_models(**kw):
    cfg = micro_cfg(**kw)
    W = sw.model_weights(cfg, gain_std=0.2)
    return cfg, Target(cfg.target, W, taps=cfg.drafter.taps), Drafter(cfg.target, cfg.drafter, W)


@pytest.mark.parametrize("rowwise", [True, False])
def test_greedy_spec_equals_greedy_ar_tiny(rowwise):
    cfg, tg, dr, prompt = tiny_models(rowwise)
    g = Sampling(0.0, 0, 1.0, 1)
    ar = ar_generate(tg, prompt, cfg.gen_len, g)
    st = SpecDecoder(tg, dr, cfg.drafter.block_size, g).generate(prompt, cfg.gen_len)
    assert st.out == ar and len(ar) == cfg.gen_len


def test_greedy_spec_with_oracle_drafts_accepts_whole_blocks():
    """Planted drafts equal to the greedy stream are all accepted: tau = B every step."""
    cfg, tg, dr, prompt = tiny_models()
    g = Sampling(0.0, 0, 1.0, 1)
    B = cfg.drafter.block_size
    ar = np.array(ar_generate(tg, prompt, cfg.gen_len + B, g))
    P = len(prompt)
    stream = np.concatenate([np.asarray(prompt), ar])  # stream[t] = token at absolute position t

    def planted(st):
        return list(stream[st.n + 1:st.n + B])

    st = SpecDecoder(tg, dr, B, g).generate(prompt, cfg.gen_len, draft_fn=planted)
    assert st.out == list(ar[:cfg.gen_len])
    assert all(t == B for t in st.taus[1:-1])
    assert P + len(st.out) >= cfg.gen_len


def test_block_size_one_sampled_equals_ar_sampling_bitwise():
    cfg, tg, dr, prompt = tiny_models()
    s = Sampling.of(cfg.sampling)
    ar = ar_generate(tg, prompt, 40, s)
    d1 = Drafter(cfg.target, replace(cfg.drafter, block_size=1), sw.model_weights(cfg, gain_std=0.1))
    st = SpecDecoder(tg, d1, 1, s).generate(prompt, 40)
    assert st.out == ar


def test_kv_rollback_matches_ar_cache():
    """After every step the committed part of the target cache equals the cache that plain decoding
    builds from the same tokens (bitwise in row-wise mode)."""
    cfg, tg, dr, prompt = tiny_models(rowwise=True)
    s = Sampling.of(cfg.sampling)
    dec = SpecDecoder(tg, dr, cfg.drafter.block_size, s)
    st = dec.new_state()
    dec.step(st, prompt=prompt)
    for _ in range(6):
        dec.step(st)
        ref = tg.new_cache()
        toks = list(prompt) + st.out[:-1]  # committed tokens 0 .. n-1 (the anchor is not yet cached)
        assert len(toks) == st.n
        for i, t in enumerate(toks):
            tg.forward(ref, [t], i, logit_rows=1)
        for l in range(cfg.target.layers):
            assert np.array_equal(ref.k[l][:st.n], st.tcache.k[l][:st.n])
            assert np.array_equal(ref.v[l][:st.n], st.tcache.v[l][:st.n])


@pytest.mark.parametrize("block", [2, 3, 4])
@pytest.mark.parametrize("sampling", [Sampling(1.0, 4, 0.9, 1), Sampling(0.8, 0, 1.0, 1), Sampling(0.0, 0, 1.0, 1)])
def test_exact_law_equality(block, sampling):
    """Brute-force enumeration: the law of the first 4 speculative tokens equals plain decoding's."""
    cfg, tg, dr = micro_models(block=block)
    prompt = [1, 3]
    k = 4
    la = ar_law(tg, prompt, k, sampling)
    ls = spec_law(SpecDecoder(tg, dr, block, sampling), prompt, k)
    assert abs(sum(la.values()) - 1.0) < 1e-12 and abs(sum(ls.values()) - 1.0) < 1e-12
    keys = set(la) | set(ls)
    assert max(abs(la.get(x, 0.0) - ls.get(x, 0.0)) for x in keys) <= 1e-12
    assert len(la) > 1 or sampling.temperature == 0.0


def test_exact_law_equality_with_good_drafts():
    """Same, with drafts that are often right (the target's own argmax), so accept branches are deep."""
    cfg, tg, dr = micro_models(block=4)
    prompt = [2, 0]
    sp = Sampling(1.0, 3, 0.95, 1)
    dec = SpecDecoder(tg, dr, 4, sp)

    def oracle_drafts(st):
        toks = list(prompt) + st.out
        out = []
        for _ in range(3):
            z, _ = tg.forward(tg.new_cache(), toks, 0, logit_rows=1)
            out.append(int(np.argmax(z[-1])))
            toks.append(out[-1])
        return out

    law_ar = ar_law(tg, prompt, 4, sp)
    law = {}

    from oracle.sampling import decide_law

    def rec(st, prob, first):
        if len(st.out) >= 4:
            key = tuple(st.out[:4])
            law[key] = law.get(key, 0.0) + prob
            return
        tokens, drafts = dec.block(st, prompt if first else None, None if first else oracle_drafts)
        logits, feats = dec.verify(st, tokens, drafts)
        for em, pe in decide_law(dec.rows(logits, exact=True), drafts):
            if pe > 0:
                s2 = st.copy()
                dec.commit(s2, tokens, drafts, em, feats)
                rec(s2, prob * pe, False)

    rec(dec.new_state(), 1.0, True)
    keys = set(law_ar) | set(law)
    assert max(abs(law_ar.get(x, 0.0) - law.get(x, 0.0)) for x in keys) <= 1e-12


def test_sampled_loop_law_monte_carlo():
    """The sampling loop itself (uniforms, filter, decide) reproduces the plain-decoding law (chi-square)."""
    cfg, tg, dr = micro_models(block=3)
    prompt = [1, 3]
    sp = Sampling(1.0, 4, 0.9, 1)
    law = ar_law(tg, prompt, 2, sp)
    counts = {}
    N = 1500
    for r in range(N):
        st = SpecDecoder(tg, dr, 3, sp, request=r).generate(prompt, 2)
        key = tuple(st.out)
        counts[key] = counts.get(key, 0) + 1
    assert set(counts) <= set(law)
    keys = sorted(law)
    obs = np.array([counts.get(k, 0) for k in keys], dtype=float)
    exp = np.array([law[k] for k in keys]) * N
    big = exp >= 5
    obs2 = np.append(obs[big], obs[~big].sum())
    exp2 = np.append(exp[big], exp[~big].sum())
    if exp2[-1] == 0:
        obs2, exp2 = obs2[:-1], exp2[:-1]
    assert scipy.stats.chisquare(obs2, exp2 * obs2.sum() / exp2.sum()).pvalue > 1e-4


@pytest.mark.parametrize("rate", [0.1, 0.3, 0.6])
def test_planted_drafter_mean_acceptance_closed_form(rate):
    """Greedy verification of drafts corrupted independently per position at rate r:
    E[tau] = sum_{j<B} (1-r)^j = (1 - (1-r)^B) / r, and the output is still the greedy stream."""
    cfg, tg, dr, prompt = tiny_models()
    g = Sampling(0.0, 0, 1.0, 1)
    B = cfg.drafter.block_size
    n_tok = 300
    ar = np.array(ar_generate(tg, prompt, n_tok + B, g))
    stream = np.concatenate([np.asarray(prompt), ar])
    V, mask = cfg.target.vocab, cfg.drafter.mask_id

    def planted(st):
        return list(sw.planted_drafts(stream, st.n, B - 1, V, mask, rate))

    st = SpecDecoder(tg, dr, B, g).generate(prompt, n_tok, draft_fn=planted)
    assert st.out == list(ar[:n_tok])
    taus = np.array(st.taus[1:-1])
    expect = (1 - (1 - rate) ** B) / rate
    var = sum((2 * j + 1) * (1 - rate) ** j for j in range(B)) - expect ** 2
    assert abs(taus.mean() - expect) < 4.5 * np.sqrt(var / len(taus)), (taus.mean(), expect)


@pytest.mark.parametrize("block", [2, 3])
@pytest.mark.parametrize("sampling", [Sampling(1.0, 4, 0.9, 1), Sampling(0.8, 3, 1.0, 1)])
def test_exact_law_equality_stochastic_drafts(block, sampling):
    """Brute-force enumeration with stochastic drafts (every draw of every draft, then every accept /
    reject outcome): the law of the first 4 tokens equals plain decoding's."""
    cfg, tg, dr = micro_models(vocab=5, block=block)
    prompt = [1, 3]
    la = ar_law(tg, prompt, 4, sampling)
    ls = spec_law(SpecDecoder(tg, dr, block, sampling, stochastic=True), prompt, 4)
    assert abs(sum(ls.values()) - 1.0) < 1e-12
    keys = set(la) | set(ls)
    assert max(abs(la.get(x, 0.0) - ls.get(x, 0.0)) for x in keys) <= 1e-12


def test_stochastic_loop_runs_and_emits_requested_length():
    cfg, tg, dr = micro_models(block=3)
    dec = SpecDecoder(tg, dr, 3, Sampling(1.0, 4, 0.9, 3), stochastic=True)
    st = dec.generate([1, 3], 12)
    assert len(st.out) == 12 and all(1 <= t <= 3 for t in st.taus)
