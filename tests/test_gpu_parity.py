"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Tolerances: logits rel-err (max |g - o| / max |o| per row) <= 1e-4 for fp32 models and <= 2e-2 for
bf16 models.  Token decisions are compared bit-exactly where both sides take them from the same
fp32 numbers (the decide stage given the device's candidates; the filter given the device's
logits); decisions the oracle takes from its own logits may differ only at flagged near-ties.
"""
import numpy as np
import pytest
import torch

import synth
from harness import (OracleFollower, StepReport, _variant, engine, log, near_tie_argmax, rel_err_rows, run_e2e,
                     run_e2e_batched, samp, small_short, tol_of, torch_weights)
from oracle.sampling import decide, decide_q, sample_dist
from oracle.spec import Sampling as OSampling
from oracle.spec import SpecDecoder, ar_generate
from synth import weights as sw

pytestmark = pytest.mark.gpu


CASES = {
    "tiny": lambda: synth.TINY,
    "small": lambda: small_short(),
    "tiny_bf16": lambda: _variant(synth.TINY, dtype="bf16"),
    "small_fp32": lambda: _variant(small_short(32), dtype="fp32"),
    "small_p300": lambda: small_short(300),
    # more than 256 pages of keys: the prefill attention reads its block-table entries chunk by chunk
    "tiny_bf16_p4200": lambda: _variant(synth.TINY, dtype="bf16", prompt_len=4200),
}


@pytest.mark.parametrize("name", ["tiny", "small", "tiny_bf16", "small_fp32", "small_p300", "tiny_bf16_p4200"])
def test_prefill_logits_and_features(name):
    cfg = CASES[name]()
    log(f"[prefill] {name}")
    W = sw.model_weights(cfg, gain_std=0.1)
    tol = tol_of(cfg)
    P = cfg.prompt_len
    eng = engine(cfg, W)
    eng.kv_alloc(0, P + 64)
    prompt = sw.prompt_ids(cfg.target.vocab, cfg.drafter.mask_id, P, 0)
    toks = torch.from_numpy(prompt).to("cuda")
    logits = torch.empty(P * cfg.target.vocab, dtype=torch.float32, device="cuda")
    eng.verify([0], toks, P, True, P, logits=logits)
    eng.status()
    g = logits.view(P, -1).cpu().numpy()
    gf = eng.features(P).cpu().numpy()
    fol = OracleFollower(cfg, W, request=0)
    z, feats = fol.prefill(prompt)
    e = rel_err_rows(g, z)
    ef = rel_err_rows(gf.reshape(P, -1), feats.reshape(P, -1))
    log(f"  logits rel-err max {e.max():.3e} mean {e.mean():.3e}; features rel-err max {ef.max():.3e}")
    assert e.max() <= tol
    assert ef.max() <= (1e-4 if cfg.target.dtype == "fp32" else 2e-2)


def _hd128_bf16(prompt_len):
    """A narrow bf16 model at head_dim 128 with a GQA group of 4 (8 q / 2 kv heads)."""
    from dataclasses import replace
    t = replace(synth.TINY.target, hidden=256, q_heads=8, kv_heads=2, head_dim=128, ffn=512, dtype="bf16")
    return replace(synth.TINY, target=t, prompt_len=prompt_len)


@pytest.mark.parametrize("P,P2,batch", [(300, 0, 1), (1100, 0, 1), (200, 0, 3), (257, 150, 2)])
def test_flash_prefill_attention(P, P2, batch):
    """Prefill-sized calls of a bf16 model at head_dim 128, which take the flash-style prefill attention
    (128-row query blocks, 64-key blocks, causal masking on the diagonal blocks): ragged last blocks
    (300 = 2 x 128 + 44), more than 1024 keys, several prompts in one call (slots given out of order, so
    each sequence reads its own page list), and a second 150-row call at positions P .. P + 149 over the
    cached prefix.  Every row's logits against the oracle within the bf16 tolerance."""
    cfg = _hd128_bf16(P)
    log(f"[flash prefill] P {P} then {P2}, batch {batch}")
    W = sw.model_weights(cfg, gain_std=0.1)
    V, tol = cfg.target.vocab, tol_of(cfg)
    eng = engine(cfg, W, max_slots=batch, max_rows=batch * max(P, P2),
                 max_pages_per_seq=(P + P2 + 64) // 16 + 2)
    assert batch * P > batch * cfg.drafter.block_size  # prefill-sized, not a decode-sized call
    for b in range(batch):
        eng.kv_alloc(b, P + P2 + 32)
    slots = list(reversed(range(batch)))
    prompts = np.stack([sw.prompt_ids(V, cfg.drafter.mask_id, P, 7 + b) for b in range(batch)])
    logits = torch.empty(batch * max(P, P2) * V, dtype=torch.float32, device="cuda")
    tp = torch.from_numpy(prompts.astype(np.int32)).to("cuda")
    eng.verify(slots, tp, P, True, P, logits=logits)
    eng.status()
    g = logits[:batch * P * V].view(batch, P, V).cpu().numpy()
    fols = [OracleFollower(cfg, W, request=b) for b in range(batch)]
    worst = 0.0
    for b in range(batch):
        z, _ = fols[b].prefill(prompts[b])
        worst = max(worst, float(rel_err_rows(g[b], z).max()))
    if P2:
        g2 = sw.prompt_ids(V, cfg.drafter.mask_id, P2, 99)
        chunk = np.stack([np.roll(g2, b) for b in range(batch)])
        eng.prefill(slots, tp, [samp(synth.GREEDY)] * batch)  # the same prompts, committed
        eng.verify(slots, torch.from_numpy(chunk.astype(np.int32)).to("cuda"), P2, False, P2, logits=logits)
        eng.status()
        g = logits[:batch * P2 * V].view(batch, P2, V).cpu().numpy()
        for b in range(batch):
            z, _ = fols[b].t.forward(fols[b].tc, list(chunk[b]), P, logit_rows=P2)
            worst = max(worst, float(rel_err_rows(g[b], z).max()))
    log(f"  logits rel-err max {worst:.3e}")
    assert worst <= tol


@pytest.mark.parametrize("name", ["tiny", "small"])
@pytest.mark.parametrize("mode", ["greedy", "sampled"])
def test_e2e_teacher_forced(name, mode):
    cfg = CASES[name]()
    log(f"[e2e] {name} {mode}")
    W = sw.model_weights(cfg, gain_std=0.1)
    sp = synth.GREEDY if mode == "greedy" else cfg.sampling
    n_tok = 64 if name == "tiny" else 24
    stream, rep, prompt = run_e2e(cfg, W, sp, n_tok)
    tol = tol_of(cfg)
    le, de = np.array(rep.logits_err), np.array(rep.draft_err)
    log(f"  logits err max {le.max():.3e}, draft logits err max {de.max():.3e}, flagged {rep.flagged}/"
        f"{rep.positions}, draft flagged {rep.draft_flagged} mismatched {rep.draft_mismatch}, taus {rep.taus}")
    assert le.max() <= tol and de.max() <= tol
    assert rep.draft_mismatch == 0
    if mode == "greedy" and name == "tiny":
        from oracle.model import Target
        tg = Target(cfg.target, W, taps=cfg.drafter.taps)
        ar = ar_generate(tg, prompt, n_tok, OSampling(0.0, 0, 1.0, 1))
        assert stream == ar


@pytest.mark.parametrize("variant", ["separate_post", "last_arriver", "one_page_splits", "uneven_splits", "no_splits",
                                     "long_no_splits", "gemm_one_tile_per_wg", "gemm_stream_k_all",
                                     "prefill_row_chunks"])
@pytest.mark.parametrize("name", ["tiny", "small"])
def test_e2e_kernel_variants(name, variant, monkeypatch):
    """The non-default kernel variants match the oracle like the defaults.  Attention (default: q / k / v
    post-processed inside attention, ~9-page key splits merged by a second kernel): a separate
    post-processing kernel; the in-kernel merge by the last split to finish; one-page splits (on the
    small model with a 320-token prompt: more than 16 splits, the merge kernel's general path); five-page
    splits (a shorter last split); a single split (no merge: the batched-call policy when the batch
    alone fills the GPU), also over a 4200-token context (more than 256 pages in one range: block-table
    entries read chunk by chunk).
    Projections (default: stream-K for the residual + norm and SwiGLU projections at M <= 16, one tile
    per work-group elsewhere): one tile per work-group everywhere; stream-K wherever the shape allows
    (q/k/v, LM heads, drafter k/v too).  Prefill (default: the tiled large-M kernel for bf16 prompts of
    128+ rows): the row-chunked kernels."""
    monkeypatch.setenv("DFLASH_ATTN_FUSED", "0" if variant == "separate_post" else "1")
    monkeypatch.setenv("DFLASH_ATTN_MERGE", "1" if variant == "last_arriver" else "0")
    monkeypatch.setenv("DFLASH_ATTN_PPS", {"one_page_splits": "1", "uneven_splits": "5"}.get(variant, "0"))
    monkeypatch.setenv("DFLASH_ATTN_WG", "1" if variant in ("no_splits", "long_no_splits") else "512")
    monkeypatch.setenv("DFLASH_GEMM_SK", {"gemm_one_tile_per_wg": "0", "gemm_stream_k_all": "1"}.get(variant, "-1"))
    monkeypatch.setenv("DFLASH_GEMM_MM", "0" if variant == "prefill_row_chunks" else "1")
    long_keys = variant in ("one_page_splits", "uneven_splits", "no_splits") and name == "small"
    cfg = small_short(prompt_len=320) if long_keys else CASES[name]()
    if variant == "long_no_splits":  # more than 256 key pages in one work-group's range
        if name != "tiny":
            pytest.skip("the tiny model covers it (a small-model oracle at 4200 tokens takes minutes)")
        cfg = _variant(synth.TINY, dtype="bf16", prompt_len=4200)
    log(f"[e2e kernel variant] {name} {variant}")
    W = sw.model_weights(cfg, gain_std=0.1)
    stream, rep, prompt = run_e2e(cfg, W, cfg.sampling, 24)
    tol = tol_of(cfg)
    le, de = np.array(rep.logits_err), np.array(rep.draft_err)
    log(f"  logits err max {le.max():.3e}, draft logits err max {de.max():.3e}")
    assert le.max() <= tol and de.max() <= tol
    assert rep.draft_mismatch == 0


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_gpu_greedy_spec_equals_gpu_greedy_ar(name):
    """Greedy speculative decoding on the device emits exactly the device's own greedy AR stream."""
    cfg = CASES[name]()
    log(f"[greedy spec == AR] {name}")
    W = sw.model_weights(cfg)
    P, B, V = cfg.prompt_len, cfg.drafter.block_size, cfg.target.vocab
    n_tok = 48
    prompt = torch.from_numpy(sw.prompt_ids(V, cfg.drafter.mask_id, P, 0)).to("cuda")
    g = samp(synth.GREEDY)
    eng = engine(cfg, W)
    eng.kv_alloc(0, P + n_tok + 2 * B)
    eng.prefill([0], prompt.view(1, -1), [g])
    ar = [int(eng.out[0].item())]
    while len(ar) < n_tok:
        eng.ar_step([0], [g])
        ar.append(int(eng.out[0].item()))
    eng.prefill([0], prompt.view(1, -1), [g])
    spec = [int(eng.out[0].item())]
    taus = []
    while len(spec) < n_tok:
        eng.spec_step([0], [g])
        tau = int(eng.n_out[0].item())
        taus.append(tau)
        spec.extend(int(x) for x in eng.out[:tau].cpu().numpy())
    eng.status()
    log(f"  taus {taus[:20]}")
    assert spec[:n_tok] == ar


def test_sampler_chi_square_and_bitexact():
    """Device accept/resample with planted drafts over many draws: decisions are bit-exact with the
    oracle's rule applied to the device's candidates; the acceptance rate of a draft x is p(x) and the
    rejection resample follows p without x (chi-square); candidate filter matches the oracle's."""
    import scipy.stats
    cfg = synth.TINY
    W = sw.model_weights(cfg)
    V, B = cfg.target.vocab, cfg.drafter.block_size
    S = 64
    eng = engine(cfg, W, max_slots=S, max_rows=S * B)
    for s_ in range(S):
        eng.kv_alloc(s_, 4 * B)
    rng = np.random.default_rng(5)
    # a fixed row distribution concentrated on 8 tokens, the rest far below
    base = np.full(V, -30.0, dtype=np.float32)
    hot = rng.choice(V, 8, replace=False)
    base[hot] = rng.normal(0, 1.0, 8).astype(np.float32)
    sp = synth.SamplingCfg(temperature=1.0, top_k=6, top_p=0.9, seed=0)
    ids_o, p_o = sample_dist(base, 1.0, 6, 0.9)
    x = int(ids_o[1])  # a mid-rank draft
    logits = torch.from_numpy(np.tile(base, S * B)).to("cuda")
    block = torch.full((S * B,), x, dtype=torch.int32, device="cuda")
    toks = torch.zeros(S * B, dtype=torch.int32, device="cuda")
    acc = 0
    resample = np.zeros(V)
    draws = 0
    for call in range(60):
        samplings = [samp(synth.SamplingCfg(1.0, 6, 0.9, 1000 * call + s_)) for s_ in range(S)]
        eng.verify(list(range(S)), toks, B, True, B)
        eng.accept(list(range(S)), B - 1, samplings, block=block, cands=True, logits=logits)
        out = eng.out[:S * B].view(S, B).cpu().numpy()
        nout = eng.n_out[:S].cpu().numpy()
        gi_all = eng.cand_ids[:S * B * 256].view(S * B, 256).cpu().numpy()
        gp_all = eng.cand_p[:S * B * 256].view(S * B, 256).cpu().numpy()
        gi, gp = gi_all[0], gp_all[0]
        k = int((gi >= 0).sum())
        assert np.array_equal(gi[:k], ids_o) and np.abs(gp[:k] - p_o).max() <= 2e-6
        assert (gi_all == gi).all() and (gp_all == gp).all()
        rows = [(gi[:k].astype(np.int64), gp[:k])] * B
        for s_ in range(S):
            tau = int(nout[s_])
            want = decide(rows, [x] * (B - 1), 0, 1000 * call + s_, s_)
            assert want == list(out[s_, :tau]), (call, s_, want, out[s_, :tau])
            draws += 1
            if tau == 1:
                resample[out[s_, 0]] += 1
            else:
                acc += 1
    px = float(p_o[list(ids_o).index(x)])
    z = (acc / draws - px) / np.sqrt(px * (1 - px) / draws)
    log(f"  accept rate {acc / draws:.4f} vs p(x) {px:.4f} (z {z:.2f}); resample counts {resample[hot]}")
    assert abs(z) < 4.5
    r = np.zeros(V)
    r[ids_o] = p_o
    r[x] = 0
    r /= r.sum()
    sup = r > 0
    assert resample[~sup].sum() == 0
    assert scipy.stats.chisquare(resample[sup], r[sup] * resample.sum()).pvalue > 1e-4


def test_candidate_filter_paths():
    """The sampler's candidate filter on planted logits over a 151936-token vocabulary (38 chunks of 4000
    per row), against the oracle filter row by row: ids exact, probabilities within 2e-6.  Covers the
    chunk shortcut (top-k <= 64: keys ranked above a bound from the waves' lane maxima) at k = 2, 7, 20
    and 64, the radix select at k = 65, 100 and 256, rows whose keys tie heavily (values on a coarse grid:
    the shortcut's candidate set overflows and the radix select decides), equal keys straddling the k-th
    place (the lowest ids win), and a temperature that divides the logits."""
    from dataclasses import replace
    cfg = replace(synth.TINY, target=replace(synth.TINY.target, vocab=151936))
    W = sw.model_weights(cfg)
    V, B = cfg.target.vocab, cfg.drafter.block_size
    S = 8
    eng = engine(cfg, W, max_slots=S, max_rows=S * B)
    for s_ in range(S):
        eng.kv_alloc(s_, 4 * B)
    rng = np.random.default_rng(11)
    ks = [2, 7, 20, 64, 65, 100, 256, 20]
    temps = [1.0, 0.7, 1.0, 1.0, 1.3, 1.0, 1.0, 1.0]
    tops = [1.0, 0.95, 0.9, 1.0, 1.0, 0.8, 1.0, 1.0]
    z = rng.standard_normal((S * B, V)).astype(np.float32) * 2.0
    for r in range(S * B):
        kind = r % B
        if kind == 1:  # a coarse grid: thousands of equal keys
            z[r] = np.round(z[r] * 2.0) / 2.0
        elif kind == 2:  # 40 equal keys straddling the k-th place, spread over the chunks
            top = np.argsort(-z[r], kind="stable")[:8]
            z[r, top] = 12.0 + np.arange(8, dtype=np.float32)
            tie = rng.choice(np.setdiff1d(np.arange(V), top), 40, replace=False)
            z[r, tie] = 11.5
    toks = torch.zeros(S * B, dtype=torch.int32, device="cuda")
    samplings = [samp(synth.SamplingCfg(temps[i], ks[i], tops[i], i)) for i in range(S)]
    eng.verify(list(range(S)), toks, B, True, B)
    block = torch.zeros(S * B, dtype=torch.int32, device="cuda")
    eng.accept(list(range(S)), B - 1, samplings, block=block, cands=True, logits=torch.from_numpy(z).to("cuda"))
    gi_all = eng.cand_ids[:S * B * 256].view(S * B, 256).cpu().numpy()
    gp_all = eng.cand_p[:S * B * 256].view(S * B, 256).cpu().numpy()
    for r in range(S * B):
        i = r // B
        ids_o, p_o = sample_dist(z[r], temps[i], ks[i], tops[i])
        k = int((gi_all[r] >= 0).sum())
        assert k == len(ids_o), (r, ks[i], k, len(ids_o))
        assert np.array_equal(gi_all[r, :k], ids_o), (r, ks[i])
        assert np.abs(gp_all[r, :k] - p_o).max() <= 2e-6, (r, ks[i])
    log(f"  candidate filter: {S * B} rows, k in {sorted(set(ks))}, ids exact")


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_e2e_stochastic_drafts(name):
    """Stochastic drafts end to end, teacher-forced: the drafter's candidate distributions match the
    oracle's filter of the device's draft logits, each draft is the oracle's draw from them with the
    same stream-1 uniform, and the min(1, p/q) / max(0, p - q) decisions are bit-exact with the oracle's
    rule on the device's candidates; logits within tolerance of the oracle's forward."""
    cfg = CASES[name]()
    log(f"[e2e stochastic drafts] {name}")
    W = sw.model_weights(cfg, gain_std=0.1)
    sp = synth.SamplingCfg(temperature=1.0, top_k=8, top_p=0.95, seed=3)
    stream, rep, prompt = run_e2e(cfg, W, sp, 48 if name == "tiny" else 24, stochastic=True)
    tol = tol_of(cfg)
    le, de = np.array(rep.logits_err), np.array(rep.draft_err)
    log(f"  logits err max {le.max():.3e}, draft logits err max {de.max():.3e}, taus {rep.taus}")
    assert le.max() <= tol and de.max() <= tol


def test_stochastic_sampler_law():
    """dflash_accept_resample_q with caller-built draft distributions q and drafts drawn from q: the
    acceptance rate is sum_x min(p, q) (z-test), the emitted token follows p (chi-square), and every
    decision is bit-exact with the oracle's rule on the device's candidates."""
    import scipy.stats
    from oracle.sampling import sample_draft
    cfg = synth.TINY
    W = sw.model_weights(cfg)
    V, B = cfg.target.vocab, cfg.drafter.block_size
    S = 64
    eng = engine(cfg, W, max_slots=S, max_rows=S * B)
    for s_ in range(S):
        eng.kv_alloc(s_, 4 * B)
    rng = np.random.default_rng(8)
    base = np.full(V, -30.0, dtype=np.float32)
    hot = rng.choice(V, 8, replace=False)
    base[hot] = rng.normal(0, 1.0, 8).astype(np.float32)
    ids_o, p_o = sample_dist(base, 1.0, 6, 0.9)
    # q: another distribution over the hot tokens, with mass where p has none and vice versa
    qb = np.full(V, -30.0, dtype=np.float32)
    qb[hot] = rng.normal(0, 1.5, 8).astype(np.float32)
    qids, qp = sample_dist(qb, 1.0, 7, 1.0)
    nd = B - 1
    qi_host = np.full((S * nd, 256), -1, dtype=np.int32)
    qp_host = np.zeros((S * nd, 256), dtype=np.float32)
    qi_host[:, :len(qids)] = qids
    qp_host[:, :len(qids)] = qp
    eng.q_ids[:S * nd * 256] = torch.from_numpy(qi_host.reshape(-1)).to("cuda")
    eng.q_p[:S * nd * 256] = torch.from_numpy(qp_host.reshape(-1)).to("cuda")
    logits = torch.from_numpy(np.tile(base, S * B)).to("cuda")
    toks = torch.zeros(S * B, dtype=torch.int32, device="cuda")
    pf = np.zeros(V)
    pf[ids_o] = p_o
    qf = np.zeros(V)
    qf[qids] = qp
    acc = first_n = 0
    first = np.zeros(V)
    for call in range(60):
        seeds = [1000 * call + s_ for s_ in range(S)]
        samplings = [samp(synth.SamplingCfg(1.0, 6, 0.9, sd)) for sd in seeds]
        # drafts drawn from q (stream 1 at the draft positions 1 .. nd after an anchor at position 0)
        drafts = np.array([[sample_draft(qids, qp, seeds[s_], i, s_) for i in range(1, nd + 1)] for s_ in range(S)],
                          dtype=np.int32)
        blk = np.zeros((S, B), dtype=np.int32)
        blk[:, 1:] = drafts
        block = torch.from_numpy(blk.reshape(-1)).to("cuda")
        eng.verify(list(range(S)), toks, B, True, B)
        eng.accept(list(range(S)), nd, samplings, block=block, cands=True, logits=logits, q=True)
        out = eng.out[:S * B].view(S, B).cpu().numpy()
        nout = eng.n_out[:S].cpu().numpy()
        gi = eng.cand_ids[:256].cpu().numpy()
        gp = eng.cand_p[:256].cpu().numpy()
        k = int((gi >= 0).sum())
        assert np.array_equal(gi[:k], ids_o) and np.abs(gp[:k] - p_o).max() <= 2e-6
        rows = [(gi[:k].astype(np.int64), gp[:k])] * B
        qrows = [(qids.astype(np.int64), qp)] * nd
        for s_ in range(S):
            tau = int(nout[s_])
            want = decide_q(rows, qrows, [int(x) for x in drafts[s_]], 0, seeds[s_], s_)
            assert want == list(out[s_, :tau]), (call, s_, want, out[s_, :tau])
            first[out[s_, 0]] += 1
            first_n += 1
            acc += tau > 1
    a = float(np.minimum(pf, qf).sum())
    z = (acc / first_n - a) / np.sqrt(a * (1 - a) / first_n)
    log(f"  accept rate {acc / first_n:.4f} vs sum min(p, q) {a:.4f} (z {z:.2f})")
    assert abs(z) < 4.5
    sup = pf > 0
    assert first[~sup].sum() == 0
    assert scipy.stats.chisquare(first[sup], pf[sup] / pf[sup].sum() * first_n).pvalue > 1e-4


def test_gpu_generator_matches_cpu():
    """The synthetic-weight fill on the device equals the CPU definition bit for bit."""
    from synth import gpu as sg
    for dtype, name, shape in [("bf16", "t.L0.wq", (96, 64)), ("fp32", "d.fc", (33, 17)), ("bf16", "t.embed", (7, 5))]:
        t = torch.empty(shape, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
        sg.fill(t, name, "w", 0, 0.02, dtype)
        ref = sw.tensor(name, shape, "w", 0, 0.02, dtype)
        assert np.array_equal(t.float().cpu().numpy(), ref)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (4, 384, 128), (8, 7168, 5120), (13, 5120, 17408), (64, 256, 1024),
                                   (37, 512, 96), (100, 160, 64), (128, 256, 1024), (300, 512, 2816),
                                   (1024, 7168, 5120)])
def test_op_linear(dtype, M, N, K):
    """The projection kernel against float64 matmul of the same (storage-typed) inputs -- bf16 models: fp16
    X, bf16 weights; fp32 models: fp32 -- tiles and ragged row counts included; fp32 accumulation bounds
    the error."""
    from speculative_decoding_dflash_amd import binding as Bd
    if dtype == "bf16" and K % 32:
        pytest.skip("bf16 needs K % 32 == 0")
    rng = np.random.default_rng(M * 7 + N + K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    xt = torch.from_numpy(x).to(torch.float16 if dtype == "bf16" else torch.float32).cuda()
    wt = torch.from_numpy(w).to(torch.bfloat16 if dtype == "bf16" else torch.float32).cuda()
    y = torch.zeros(M * N, dtype=torch.float32, device="cuda")
    Bd.dflash_op_linear(Bd.BF16 if dtype == "bf16" else Bd.F32, M, N, K, xt, wt, y)
    torch.cuda.synchronize()
    ref = xt.double().cpu().numpy() @ wt.double().cpu().numpy().T
    got = y.view(M, N).cpu().numpy()
    err = np.abs(got - ref).max() / np.abs(ref).max()
    log(f"  linear {dtype} {M}x{N}x{K}: rel err {err:.2e}")
    assert err < 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("M,N,K", [(1, 5120, 5120), (8, 5120, 17408), (13, 34816, 5120), (16, 640, 256),
                                   (5, 5120, 25600), (8, 96, 128)])
def test_op_linear_sk(dtype, M, N, K):
    """The stream-K projection kernel on its own (dflash_op_linear_sk, caller scratch): against float64
    matmul of the same storage-typed inputs, and twice in a row on one scratch block (the counters the
    first call leaves are cleared by the second), at 27B decode shapes, a ragged row count and a shape
    with fewer items than work-groups."""
    from speculative_decoding_dflash_amd import binding as Bd
    rng = np.random.default_rng(M * 13 + N + K)
    xt = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32))
    xt = xt.to(torch.float16 if dtype == "bf16" else torch.float32).cuda()
    wt = torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    wt = wt.to(torch.bfloat16 if dtype == "bf16" else torch.float32).cuda()
    scratch = torch.empty(Bd.dflash_op_linear_sk_scratch_bytes(N), dtype=torch.uint8, device="cuda")
    ys = [torch.zeros(M * N, dtype=torch.float32, device="cuda") for _ in range(2)]
    for y in ys:
        Bd.dflash_op_linear_sk(Bd.BF16 if dtype == "bf16" else Bd.F32, M, N, K, xt, wt, y, scratch)
    torch.cuda.synchronize()
    ref = xt.double().cpu().numpy() @ wt.double().cpu().numpy().T
    got = ys[0].view(M, N).cpu().numpy()
    err = np.abs(got - ref).max() / np.abs(ref).max()
    log(f"  stream-K linear {dtype} {M}x{N}x{K}: rel err {err:.2e}")
    assert err < 1e-5
    assert torch.equal(ys[0], ys[1])


@pytest.mark.parametrize("M,N,K,ranges", [(1, 128, 64, 1), (37, 96, 192, 1), (200, 640, 256, 1), (64, 5120, 5120, 8),
                                          (256, 7168, 5120, 8), (256, 5120, 17408, 8), (256, 34816, 5120, 1),
                                          (1000, 1024, 1024, 1), (130, 5120, 64, 1), (256, 151936, 5120, 1)])
def test_op_linear_f16x(M, N, K, ranges):
    """The tiled fp16 projection kernel of large calls (dflash_op_linear_f16x) against float64 matmul of
    the same fp16 X and bf16 weights (converted exactly inside the kernel): tile tails in rows and
    columns, one K step, 27B decode-batch shapes with K ranges (summed here in range order) and the
    27B LM head.  Sampled rows at the largest shapes."""
    from speculative_decoding_dflash_amd import binding as Bd
    rng = np.random.default_rng(M * 31 + N + K)
    xt = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.float16).cuda()
    wt = torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16).cuda()
    y = torch.full((ranges * M * N,), float("nan"), dtype=torch.float32, device="cuda")
    got_r = Bd.dflash_op_linear_f16x(M, N, K, xt, wt, y, ranges)
    torch.cuda.synchronize()
    assert 1 <= got_r <= ranges
    if ranges > 1 and M * N >= 256 * 5120:
        assert got_r > 1, "a decode-batch shape with few tiles should split K"
    parts = y.view(ranges, M, N)[:got_r]
    tot = parts[0].clone()
    for z in range(1, got_r):
        tot += parts[z]
    rows = np.arange(M) if M * N <= 1 << 22 else np.unique(rng.integers(0, M, 24))
    ref = xt[rows].double().cpu().numpy() @ wt.double().cpu().numpy().T
    got = tot[rows].cpu().numpy()
    assert np.isfinite(got).all()
    err = np.abs(got - ref).max() / np.abs(ref).max()
    log(f"  f16x linear {M}x{N}x{K}: {got_r} K ranges, rel err {err:.2e}")
    assert err < 1e-5


@pytest.mark.parametrize("stochastic", [False, True])
@pytest.mark.parametrize("name", ["tiny", "small"])
def test_graph_replay_equals_eager_steps(name, stochastic):
    """A speculative step captured into a HIP graph and replayed performs exactly the eager steps: same
    emitted tokens, acceptance counts, drafts and logits at every replay, with eager work and device
    synchronisation between the replays (argmax drafts and stochastic drafts)."""
    cfg = CASES[name]()
    log(f"[graph replay] {name} stochastic={stochastic}")
    W = sw.model_weights(cfg)
    P, B, V = cfg.prompt_len, cfg.drafter.block_size, cfg.target.vocab
    steps = 6
    prompt = torch.from_numpy(sw.prompt_ids(V, cfg.drafter.mask_id, P, 0)).to("cuda")
    s = samp(cfg.sampling)

    def run(use_graph):
        eng = engine(cfg, W)
        eng.kv_alloc(0, P + (steps + 2) * B)
        eng.prefill([0], prompt.view(1, -1), [s])
        eng.spec_step([0], [s], stochastic=stochastic)  # a capture needs the steady state (a block verify)
        g = eng.capture_spec_step([0], [s], stochastic=stochastic) if use_graph else None
        rec = []
        for _ in range(steps):
            if g is not None:
                g.replay()
            else:
                eng.spec_step([0], [s], stochastic=stochastic)
            torch.cuda.synchronize()
            n = int(eng.n_out[0])
            rec.append((n, eng.out[:n].cpu().clone(), eng.block[:B].cpu().clone(), eng.logits[: B * V].cpu().clone()))
        eng.status()
        return rec

    eager, graph = run(False), run(True)
    for i, (a, b) in enumerate(zip(eager, graph)):
        assert a[0] == b[0], f"step {i}: n_out {a[0]} vs {b[0]}"
        assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2]), f"step {i}: tokens or drafts differ"
        assert torch.equal(a[3], b[3]), f"step {i}: logits differ"


def test_graph_capture_needs_steady_state():
    """A captured step replays the drafter injection with the row count and feature stride of the verify
    that preceded the capture, so a capture right after a prefill (prompt-length rows) or after a plain
    decoding step (one row) is refused; captured after one eager step, at batch 2 and with a page budget
    that just fits the run, the replays equal the eager steps bit for bit (tokens, acceptance counts,
    drafts) and raise no device error (the injection's padding rows past the committed ones are neither
    written nor checked)."""
    cfg = _variant(synth.TINY, prompt_len=96)
    W = sw.model_weights(cfg)
    P, B, V = cfg.prompt_len, cfg.drafter.block_size, cfg.target.vocab
    steps = 5
    prompts = torch.stack([torch.from_numpy(sw.prompt_ids(V, cfg.drafter.mask_id, P, r)) for r in range(2)]).to("cuda")
    s = samp(cfg.sampling)
    slots = [0, 1]

    def new_engine():
        eng = engine(cfg, W, max_slots=2, max_rows=2 * P, max_pages_per_seq=(P + (steps + 3) * B) // 16 + 1)
        for r in slots:
            eng.kv_alloc(r, P + (steps + 3) * B)
        return eng

    eng = new_engine()
    eng.prefill(slots, prompts, [s, s])
    with pytest.raises(RuntimeError, match="block verify"):
        eng.capture_spec_step(slots, [s, s])
    eng.ar_step(slots, [s, s])
    with pytest.raises(RuntimeError, match="block verify"):
        eng.capture_spec_step(slots, [s, s])
    eng.close()

    def run(use_graph):
        eng = new_engine()
        eng.prefill(slots, prompts, [s, s])
        eng.spec_step(slots, [s, s])
        g = eng.capture_spec_step(slots, [s, s]) if use_graph else None
        out = []
        for _ in range(steps):
            if g is not None:
                g.replay()
            else:
                eng.spec_step(slots, [s, s])
            n = eng.n_out[:2].cpu().clone()
            out.append((n, eng.out[:2 * B].view(2, B).cpu().clone(), eng.block[:2 * B].cpu().clone()))
        eng.status()  # raises on any device-side flag
        eng.close()
        return out

    eager, graph = run(False), run(True)
    for i, (a, b) in enumerate(zip(eager, graph)):
        assert torch.equal(a[0], b[0]), f"step {i}: n_out {a[0]} vs {b[0]}"
        for r in slots:
            n = int(a[0][r])
            assert torch.equal(a[1][r, :n], b[1][r, :n]), f"step {i} slot {r}: tokens differ"
        assert torch.equal(a[2], b[2]), f"step {i}: drafts differ"


_LENS24 = (40, 17, 96, 33, 64, 9, 120, 75, 50, 28, 101, 66, 12, 88, 45, 70, 31, 58, 110, 23, 77, 6, 92, 49)


@pytest.mark.parametrize("name,lens,mode,rows_path", [
    ("tiny", (32, 9, 21, 32), "sampled", "default"),
    ("small", (128, 37, 90, 61), "greedy", "default"),
    ("small", (53, 128, 7, 100, 64, 31, 128, 80), "sampled", "default"),
    ("small", (53, 128, 7, 100, 64, 31, 128, 80), "sampled", "row_chunks"),
    ("small", (40, 17, 96, 33, 64, 9, 120, 75, 50, 28, 101, 66, 12, 88, 45, 70), "greedy", "default"),
    ("small", _LENS24, "sampled", "default")])
def test_e2e_batched_ragged(name, lens, mode, rows_path, monkeypatch):
    """Batched steps over requests at different lengths match each request's oracle like the batch-1
    runs.  Rows M = batch x block: 16 (tiny, fp32: row-chunk kernels), 32, 64 and 128 (bf16: all rows in
    one tiled launch with 64- or 128-row tiles, K split over work-groups and the ranges reduced in
    order by the epilogue kernel), 64 again on the row-chunk kernels (DFLASH_GEMM_MB=0), and 192 rows
    (two 128-row tiles, the second partial)."""
    monkeypatch.setenv("DFLASH_GEMM_MB", "0" if rows_path == "row_chunks" else "1")
    cfg = CASES[name]()
    log(f"[e2e batched] {name} {mode} prompts {lens}")
    W = sw.model_weights(cfg, gain_std=0.1)
    sp = synth.GREEDY if mode == "greedy" else cfg.sampling
    reps = run_e2e_batched(cfg, W, sp, 4, list(lens))
    tol = tol_of(cfg)
    for b, rep in enumerate(reps):
        le, de = np.array(rep.logits_err), np.array(rep.draft_err)
        log(f"  slot {b}: logits err max {le.max():.3e}, draft err max {de.max():.3e}, taus {rep.taus}")
        assert le.max() <= tol and de.max() <= tol
        assert rep.draft_mismatch == 0


def _ar_with_logits(eng, slot, prompt, n, g):
    """Device greedy plain decoding of n tokens for one slot; returns the tokens and, per token, the
    fp32 logit row that produced it (on the host)."""
    V = eng.cfg.target.vocab
    eng.prefill([slot], prompt.view(1, -1), [g])
    toks, rows = [int(eng.out[0])], [eng.logits[:V].cpu().numpy().copy()]
    while len(toks) < n:
        eng.ar_step([slot], [g])
        toks.append(int(eng.out[0]))
        rows.append(eng.logits[:V].cpu().numpy().copy())
    return toks, rows


def _fp32_target_logits(cfg, Wt, tokens, rows):
    """Independent fp32 forward of the target (torch on the GPU, bf16 weights upcast layer by layer,
    fp32 activations throughout -- no bf16 rounding anywhere): the logits at the given row indices of
    the causal forward over `tokens`.  The model as the oracle defines it: pre-norm layers with RMSNorm
    (eps), per-head q/k RMSNorm, rotate-half RoPE (fp64 angles), GQA softmax attention scaled by
    1/sqrt(d), SwiGLU, untied LM head."""
    t = cfg.target
    dev = Wt["t.embed"].device
    T, D, Hq, Hk = len(tokens), t.head_dim, t.q_heads, t.kv_heads
    ids = torch.as_tensor(np.asarray(tokens, dtype=np.int64), device=dev)

    def rms(x, g):
        return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + t.rms_eps) * g.float()

    inv = t.rope_theta ** (-2.0 * torch.arange(D // 2, dtype=torch.float64, device=dev) / D)
    ang = torch.arange(T, dtype=torch.float64, device=dev)[:, None] * inv[None]
    cos, sin = torch.cos(ang).float()[:, None], torch.sin(ang).float()[:, None]

    def rope(x):  # [T, h, D]
        a, b = x[..., :D // 2], x[..., D // 2:]
        return torch.cat([a * cos - b * sin, b * cos + a * sin], -1)

    mask = torch.ones(T, T, dtype=torch.bool, device=dev).tril()
    x = Wt["t.embed"][ids].float()
    for l in range(t.layers):
        w = lambda k: Wt[f"t.L{l}.{k}"]
        h = rms(x, w("attn_norm"))
        q = rope(rms((h @ w("wq").float().t()).view(T, Hq, D), w("q_norm")))
        k = rope(rms((h @ w("wk").float().t()).view(T, Hk, D), w("k_norm")))
        v = (h @ w("wv").float().t()).view(T, Hk, D)
        k = k.repeat_interleave(Hq // Hk, 1)
        v = v.repeat_interleave(Hq // Hk, 1)
        qh, kh, vh = q.transpose(0, 1).contiguous(), k.permute(1, 2, 0).contiguous(), v.transpose(0, 1).contiguous()
        sc = torch.matmul(qh, kh) / (D ** 0.5)  # [Hq, T, T]
        sc = sc.masked_fill(~mask, float("-inf"))
        a = torch.matmul(torch.softmax(sc, -1), vh).transpose(0, 1).reshape(T, Hq * D)
        x = x + a @ w("wo").float().t()
        h = rms(x, w("ffn_norm"))
        x = x + (torch.nn.functional.silu(h @ w("w_gate").float().t()) * (h @ w("w_up").float().t())) @ \
            w("w_down").float().t()
    h = rms(x[list(rows)], Wt["t.final_norm"])
    return (h @ Wt["t.lm_head"].float().t()).cpu().numpy().astype(np.float64)


def test_fp32_forward_matches_oracle():
    """The fp32 torch forward used at the 27B shape reproduces the oracle (float64) on the small model
    with non-unit gains: logits of every prompt row within 1e-4 relative."""
    cfg = small_short(prompt_len=48, layers=2)
    W = sw.model_weights(cfg, gain_std=0.1)
    Wt = torch_weights(W, cfg)
    prompt = sw.prompt_ids(cfg.target.vocab, cfg.drafter.mask_id, cfg.prompt_len, 0)
    z, _ = OracleFollower(cfg, W, request=0).prefill(prompt)
    ref = _fp32_target_logits(cfg, Wt, prompt.tolist(), list(range(cfg.prompt_len)))
    e = rel_err_rows(ref, z)
    log(f"[fp32 forward vs oracle] max rel-err {e.max():.2e}")
    assert e.max() <= 1e-4


def _fp32_drafter_logits(cfg, Wt, feats, anchor, n):
    """Independent fp32 forward of the drafter (torch on the GPU, bf16 weights upcast, fp32 activations):
    the injected context of positions 0 .. n-1 from target features feats [n, taps, hidden] (c =
    RMSNorm(fc [taps]); per layer K = RoPE(k_norm(W_k c)), V = W_v c), then the block [anchor, MASK x
    (B-1)] at n .. n+B-1 through the drafter's layers, block keys visible to every block query, context
    key k to query p only when p - k < window (window 0: all); final norm, shared LM head on the mask
    rows.  Returns the [B-1, vocab] logits (float64, on the host)."""
    t, d = cfg.target, cfg.drafter
    dev = Wt["t.embed"].device
    D, Hq, Hk, B, Wn = t.head_dim, t.q_heads, t.kv_heads, d.block_size, d.window
    f = torch.as_tensor(feats, dtype=torch.float32, device=dev).reshape(n, -1)

    def rms(x, g):
        return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + t.rms_eps) * g.float()

    inv = t.rope_theta ** (-2.0 * torch.arange(D // 2, dtype=torch.float64, device=dev) / D)
    ang = torch.arange(n + B, dtype=torch.float64, device=dev)[:, None] * inv[None]
    cos, sin = torch.cos(ang).float()[:, None], torch.sin(ang).float()[:, None]

    def rope(x, p0):  # [T, h, D] at positions p0 ..
        c, s_ = cos[p0:p0 + len(x)], sin[p0:p0 + len(x)]
        a, b = x[..., :D // 2], x[..., D // 2:]
        return torch.cat([a * c - b * s_, b * c + a * s_], -1)

    c = rms(f @ Wt["d.fc"].float().t(), Wt["d.hidden_norm"])
    ids = torch.tensor([anchor] + [d.mask_id] * (B - 1), dtype=torch.int64, device=dev)
    x = Wt["t.embed"][ids].float()
    kpos = torch.arange(n + B, device=dev)
    qpos = torch.arange(n, n + B, device=dev)
    ctx_ok = (kpos[None] < n) & ((Wn <= 0) | (qpos[:, None] - kpos[None] < Wn))
    allowed = ctx_ok | (kpos[None] >= n)  # [B, n + B]
    for j in range(d.layers):
        w = lambda k: Wt[f"d.L{j}.{k}"]
        kc = rope(rms((c @ w("wk").float().t()).view(n, Hk, D), w("k_norm")), 0)
        vc = (c @ w("wv").float().t()).view(n, Hk, D)
        h = rms(x, w("attn_norm"))
        q = rope(rms((h @ w("wq").float().t()).view(B, Hq, D), w("q_norm")), n)
        kb = rope(rms((h @ w("wk").float().t()).view(B, Hk, D), w("k_norm")), n)
        vb = (h @ w("wv").float().t()).view(B, Hk, D)
        k = torch.cat([kc, kb]).repeat_interleave(Hq // Hk, 1)
        v = torch.cat([vc, vb]).repeat_interleave(Hq // Hk, 1)
        sc = torch.matmul(q.transpose(0, 1).contiguous(), k.permute(1, 2, 0).contiguous()) / (D ** 0.5)
        sc = sc.masked_fill(~allowed[None], float("-inf"))
        a = torch.matmul(torch.softmax(sc, -1), v.transpose(0, 1).contiguous()).transpose(0, 1).reshape(B, Hq * D)
        x = x + a @ w("wo").float().t()
        h = rms(x, w("ffn_norm"))
        x = x + (torch.nn.functional.silu(h @ w("w_gate").float().t()) * (h @ w("w_up").float().t())) @ \
            w("w_down").float().t()
    h = rms(x[1:], Wt["d.final_norm"])
    return (h @ Wt["t.lm_head"].float().t()).cpu().numpy().astype(np.float64)


def test_fp32_drafter_matches_oracle():
    """The fp32 torch drafter used at the 27B width reproduces the oracle's drafter (float64) on the
    small shape with a 24-token window over a 96-token context and non-unit gains: draft logits within
    1e-4 relative."""
    from dataclasses import replace
    from oracle.model import Drafter, Target
    cfg = small_short(prompt_len=96, layers=2)
    cfg = replace(cfg, drafter=replace(cfg.drafter, taps=(0, 1), window=24))
    W = sw.model_weights(cfg, gain_std=0.1)
    Wt = torch_weights(W, cfg)
    prompt = sw.prompt_ids(cfg.target.vocab, cfg.drafter.mask_id, cfg.prompt_len, 0)
    tg, dr = Target(cfg.target, W, taps=cfg.drafter.taps), Drafter(cfg.target, cfg.drafter, W)
    _, feats = tg.forward(tg.new_cache(), list(prompt), 0)
    dc = dr.new_cache()
    dr.inject(dc, feats, 0)
    n, anchor = cfg.prompt_len, 17
    z = dr.draft_logits(dc, anchor, n)
    ref = _fp32_drafter_logits(cfg, Wt, feats, anchor, n)
    e = rel_err_rows(ref, z)
    log(f"[fp32 drafter vs oracle] max rel-err {e.max():.2e}")
    assert e.max() <= 1e-4


def test_27b_width_drafter_vs_fp32_drafter():
    """The drafter at the full 27B width -- five taps (the fc projection over K = 25600), two layers, the
    2048-token window over a 2300-token context -- against the fp32 torch drafter fed the device's own
    target features: the draft after the prefill (the injection skips prompt rows no draft can reach
    and runs on the tiled kernel) and the draft after one speculative step (eight injected rows through
    the stream-K fc), draft logits within 2e-2, drafts equal to the reference argmax except at near
    ties."""
    from dataclasses import replace
    from speculative_decoding_dflash_amd import binding as Bd
    from speculative_decoding_dflash_amd.runner import Engine
    from synth import gpu as sg
    from synth.configs import with_layers
    base = synth.CONFIGS["27b"]
    cfg = replace(with_layers(base, 5, 2, (0, 1, 2, 3, 4)), prompt_len=2300)
    t, d = cfg.target, cfg.drafter
    P, B, V, H = cfg.prompt_len, d.block_size, t.vocab, t.hidden
    nt = len(d.taps)
    log(f"[27b-width drafter vs fp32] taps {d.taps}, {d.layers} drafter layers, window {d.window}, prompt {P}")
    Wt = sg.model_weights(cfg)
    eng = Engine(cfg, Wt, max_slots=1, max_rows=P, max_pages_per_seq=(P + 8 * B) // 16 + 4)
    eng.kv_alloc(0, P + 6 * B)
    g = samp(synth.GREEDY)
    prompt = torch.from_numpy(sw.prompt_ids(V, d.mask_id, P, 0)).to("cuda")

    def feats_of(rows):  # the device's features of the last verify, [rows, taps, H]
        return eng.features(rows).cpu().numpy()

    eng.prefill([0], prompt.view(1, -1), [g])
    ctx = feats_of(P)
    anchor, n = int(eng.out[0]), P
    worst = 0.0
    for step in range(2):
        Bd.dflash_draft_block(eng.ctx, [0], eng.feats, eng.block, eng.draft_logits)
        got = eng.draft_logits[:(B - 1) * V].view(B - 1, V).cpu().numpy()
        ref = _fp32_drafter_logits(cfg, Wt, ctx, anchor, n)
        e = rel_err_rows(got, ref)
        drafts = [int(x) for x in eng.block[1:B].cpu().numpy()]
        for i in range(B - 1):
            if drafts[i] != int(np.argmax(ref[i])):
                assert near_tie_argmax(ref[i], 2e-2), f"step {step}: draft {i} differs without a near tie"
        log(f"  draft {step} at n {n}: rel-err max {e.max():.2e}")
        worst = max(worst, float(e.max()))
        if step == 0:  # one verify + accept: its committed rows are injected by the next draft
            eng.verify([0], eng.block, B, False, B)
            eng.accept([0], B - 1, [g])
            tau = int(eng.n_out[0])
            ctx = np.concatenate([ctx, feats_of(B)[:tau]])
            anchor, n = int(eng.out[tau - 1]), n + tau
    eng.status()
    assert worst <= 2e-2
    eng.close()
    del Wt
    torch.cuda.empty_cache()


@pytest.mark.parametrize("config,layers", [("27b", 2), ("27b", 8), ("27b", 16), ("27b", 64), ("4b", 2), ("4b", 36)])
def test_width_vs_fp32_forward(config, layers):
    """The device at the full 27B width (hidden 5120, 40 q / 8 kv heads x 128, FFN 17408, vocab 151936)
    and the 4B width (hidden 2560, 32 q / 8 kv heads x 128: a GQA group of 4, FFN 9728) against an
    independent fp32 forward of the same tokens, as the depth grows: a 128-token prefill
    (tiled projections, every row's logits) and 8 plain-decoding steps (row-chunked projections, split
    decode attention).  Every depth is held to the bf16 tolerance (2e-2): the device keeps every operand
    of its matrix products other than the bf16 weights -- projection inputs, q, the KV cache, the
    softmax weights -- in fp16, so the independent roundings that accumulate over 64 random-weight
    layers stay far below it."""
    from synth import gpu as sg
    from synth.configs import with_layers
    from speculative_decoding_dflash_amd.runner import Engine
    base = synth.CONFIGS[config]
    taps = tuple(sorted({min(t, layers - 1) for t in base.drafter.taps}))
    cfg = with_layers(base, layers, 1, taps)
    from dataclasses import replace
    cfg = replace(cfg, prompt_len=128)
    t, d = cfg.target, cfg.drafter
    P, V, n = cfg.prompt_len, t.vocab, 8
    log(f"[{config} width vs fp32] {layers} layers")
    Wt = sg.model_weights(cfg)
    eng = Engine(cfg, Wt, max_slots=1, max_rows=P, max_pages_per_seq=(P + 4 * n) // 16 + 4)
    eng.kv_alloc(0, P + 2 * n)
    prompt = torch.from_numpy(sw.prompt_ids(V, d.mask_id, P, 0)).to("cuda")
    logits = torch.empty(P * V, dtype=torch.float32, device="cuda")
    eng.verify([0], prompt, P, True, P, logits=logits)
    g_pre = logits.view(P, V).cpu().numpy()
    g = samp(synth.GREEDY)
    eng.prefill([0], prompt.view(1, -1), [g])  # the same prefill, committed (one logit row)
    toks, rows = [int(eng.out[0])], []
    for _ in range(n):
        eng.ar_step([0], [g])
        rows.append(eng.logits[:V].cpu().numpy().copy())
        toks.append(int(eng.out[0]))
    eng.status()
    ref = _fp32_target_logits(cfg, Wt, prompt.cpu().numpy().tolist() + toks[:n], list(range(P + n)))
    e_pre = rel_err_rows(g_pre, ref[:P])
    e_ar = rel_err_rows(np.stack(rows), ref[P:P + n])
    log(f"  prefill rows max {e_pre.max():.2e} mean {e_pre.mean():.2e}; decode rows max {e_ar.max():.2e}")
    bound = 2e-2
    assert e_pre.max() <= bound and e_ar.max() <= bound
    del eng, Wt
    torch.cuda.empty_cache()


@pytest.mark.parametrize("conc,whole_block", [(1, False), (8, False), (32, False), (8, True)])
def test_27b_greedy_spec_equals_greedy_ar(conc, whole_block, monkeypatch):
    """At the 27B shape with a 1024-token prompt (the measured configuration at concurrency 1, and the
    batched verify / draft at concurrency 8 and 32): greedy speculative decoding emits the device's own
    greedy plain-decoding stream for every request; a stream may diverge only at a near tie of the
    plain-decoding logits; for the first 8 requests both paths' logit rows are held against an fp32
    forward of the same tokens, and the verify rows against the plain-decoding rows, within the bf16
    tolerance (the batched rows use other row tiles and key splits, so their roundings differ from
    plain decoding's).  whole_block: the batched attention work-groups hold the whole block (three
    16-wide query tiles at the 27B head ratio), as batched calls over long key ranges do."""
    if whole_block:
        monkeypatch.setenv("DFLASH_ATTN_QTILE", "8")
    _greedy_spec_vs_ar(synth.CONFIGS["27b"], conc, 16 if conc > 1 else 24)


@pytest.mark.parametrize("block", [4, 8, 16])
def test_4b_greedy_spec_equals_greedy_ar(block):
    """The 4B shape (36 layers, hidden 2560, 32 q / 8 kv heads x 128, vocab 151936) with a 2048-token
    prompt at blocks of 4, 8 and 16: the same properties as at the 27B shape."""
    from dataclasses import replace
    cfg = synth.CONFIGS["4b"]
    cfg = replace(cfg, drafter=replace(cfg.drafter, block_size=block))
    _greedy_spec_vs_ar(cfg, 1, 24)


def _greedy_spec_vs_ar(cfg, conc, n):
    from speculative_decoding_dflash_amd import binding as Bd
    from synth import gpu as sg
    t, d = cfg.target, cfg.drafter
    B, P, V = d.block_size, cfg.prompt_len, t.vocab
    log(f"[{cfg.name} greedy spec == AR] conc {conc}, block {B}")
    Wt = sg.model_weights(cfg)
    from speculative_decoding_dflash_amd.runner import Engine
    eng = Engine(cfg, Wt, max_slots=conc, max_rows=max(P, conc * B), max_pages_per_seq=(P + (n + 4) * B) // 16 + 4)
    g = samp(synth.GREEDY)
    prompts = [torch.from_numpy(sw.prompt_ids(V, d.mask_id, P, r)).to("cuda") for r in range(conc)]
    for r in range(conc):
        eng.kv_alloc(r, P + (n + 3) * B)
    ar = [_ar_with_logits(eng, r, prompts[r], n, g) for r in range(conc)]
    # speculative: each slot prefilled and primed alone, then batched verify -> accept -> draft
    spec = [[] for _ in range(conc)]
    spec_rows = [dict() for _ in range(conc)]  # position index in the stream -> verify logit row
    for r in range(conc):
        eng.prefill([r], prompts[r].view(1, -1), [g])
        spec[r].append(int(eng.out[0]))
        Bd.dflash_draft_block(eng.ctx, [r], eng.feats, eng.block[r * B:], None)
    slots = list(range(conc))
    while min(len(x) for x in spec) < n:
        eng.verify(slots, eng.block, B, False, B)
        eng.accept(slots, B - 1, [g] * conc)
        taus = eng.n_out[:conc].cpu().numpy()
        outs = eng.out[:conc * B].view(conc, B).cpu().numpy()
        logits = eng.logits[:conc * B * V].view(conc, B, V)
        for r in range(conc):
            base = len(spec[r])
            for i in range(int(taus[r])):
                if base + i < n:
                    spec_rows[r][base + i] = logits[r, i].cpu().numpy().copy()
            spec[r].extend(int(x) for x in outs[r, :int(taus[r])])
        eng.draft(slots)
    eng.status()
    tol = 2e-2
    worst_pair = worst_ar = worst_spec = 0.0
    for r in range(conc):
        a_toks, a_rows = ar[r]
        s_toks = spec[r][:n]
        k = next((i for i in range(n) if s_toks[i] != a_toks[i]), n)
        if k < n:
            z = a_rows[k]
            assert near_tie_argmax(z, tol), f"request {r}: diverges at {k} without a near tie"
        # every verify row whose prefix matches: indices up to and including the first divergence
        idx = [i for i in range(1, min(k + 1, n)) if i in spec_rows[r]]
        assert idx
        errs = [float(rel_err_rows(spec_rows[r][i][None], a_rows[i][None])[0]) for i in idx]
        msg = (f"  request {r}: {k}/{n} tokens equal, {len(errs)} verify rows compared, max rel-err vs plain "
               f"decoding {max(errs):.2e}")
        worst_pair = max(worst_pair, max(errs))
        if r < 8:  # each device path against an independent fp32 forward of the same tokens
            P_r = len(prompts[r])
            toks = prompts[r].cpu().numpy().tolist() + a_toks[:n]
            ref = _fp32_target_logits(cfg, Wt, toks, [P_r - 1 + i for i in range(n)])
            e_ar = float(rel_err_rows(np.stack(a_rows[:n]), ref).max())
            e_sp = float(rel_err_rows(np.stack([spec_rows[r][i] for i in idx]), ref[idx]).max())
            worst_ar, worst_spec = max(worst_ar, e_ar), max(worst_spec, e_sp)
            msg += f"; vs fp32 forward: plain decoding {e_ar:.2e}, speculative {e_sp:.2e}"
        log(msg)
    log(f"  worst: spec vs plain {worst_pair:.2e}, plain vs fp32 {worst_ar:.2e}, spec vs fp32 {worst_spec:.2e}")
    assert worst_ar <= tol and worst_spec <= tol and worst_pair <= tol
    del eng, Wt
    torch.cuda.empty_cache()
