"""Workload-level parity of the HIP path (through the C ABI): the drafter's sliding window over
contexts longer than the window, blocks of 16, the small model as configured (512-token prompt, 512
generated tokens, T = 1 / top-k 20 / top-p 0.95) teacher-forced against the oracle, and the
planted-drafter acceptance law on the device.

Tolerances as in test_gpu_parity: logits rel-err <= 1e-4 (fp32 models) / 2e-2 (bf16 models);
decisions bit-exact given the device's candidates; drafts equal to the oracle's argmax except at
flagged near-ties.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
from harness import (engine, log, run_e2e, run_e2e_batched, samp, small_short, tol_of)
from synth import weights as sw

pytestmark = pytest.mark.gpu


def with_window(cfg, window, prompt_len=None):
    return replace(cfg, drafter=replace(cfg.drafter, window=window), prompt_len=prompt_len or cfg.prompt_len)


def with_block(cfg, block):
    return replace(cfg, drafter=replace(cfg.drafter, block_size=block))


def _check(rep, cfg):
    tol = tol_of(cfg)
    le, de = np.array(rep.logits_err), np.array(rep.draft_err)
    log(f"  logits err max {le.max():.3e}, draft logits err max {de.max():.3e}, draft flagged {rep.draft_flagged} "
        f"mismatched {rep.draft_mismatch}, taus {rep.taus[:16]}")
    assert le.max() <= tol and de.max() <= tol
    assert rep.draft_mismatch == 0


@pytest.mark.parametrize("name", ["tiny", "small", "g5"])
def test_window_e2e_teacher_forced(name):
    """The drafter's sliding window ("结构一览" of the rytg.cn page: 2048-token sliding-window
    attention) with contexts several windows long, one request: the fused decode attention reads its
    per-query window (key ranges starting after key 0), and the injection after the prefill skips the
    prompt rows no draft can reach.  Draft logits and target logits within tolerance of the oracle
    (whose drafter masks context keys at distance >= W), drafts equal to the oracle's argmax."""
    if name == "tiny":
        cfg, n = with_window(synth.TINY, 24, prompt_len=96), 48
    elif name == "g5":
        cfg, n = g5_model(32, 200), 32
    else:
        cfg, n = with_window(small_short(320), 64), 24
    log(f"[window e2e] {name} window {cfg.drafter.window} prompt {cfg.prompt_len}")
    W = sw.model_weights(cfg, gain_std=0.1)
    _, rep, _ = run_e2e(cfg, W, cfg.sampling, n)
    _check(rep, cfg)


def g5_model(window, prompt_len):
    """A two-layer bf16 model with the 27B shape's GQA group of 5 (10 q / 2 kv heads x 64), so that a
    block of 8 spans three 16-wide query tiles, with a sliding-window drafter."""
    t = synth.DecoderCfg(layers=2, hidden=512, q_heads=10, kv_heads=2, head_dim=64, ffn=512, vocab=512,
                         rope_theta=1e6)
    d = synth.DrafterCfg(layers=1, taps=(0, 1), block_size=8, mask_id=511, window=window)
    return synth.RunCfg(name="g5", target=t, drafter=d, prompt_len=prompt_len, gen_len=64)


@pytest.mark.parametrize("model,qtile", [("small", "default"), ("g5", "default"), ("g5", "whole_block")])
def test_window_batched(model, qtile, monkeypatch):
    """Six requests decoded together with a window of 64 (small) or 32 (GQA group 5) tokens and prompts
    of 77-320 tokens: q/k/v post-processed by their own kernel and the batched attention with
    per-sequence key ranges that start after key 0; at the GQA group of 5 once with one 16-wide query
    tile per work-group (three per block) and once with work-groups holding the whole block (the layout
    batched calls take over long key ranges)."""
    if qtile == "whole_block":
        monkeypatch.setenv("DFLASH_ATTN_QTILE", "8")
    cfg = with_window(small_short(320), 64) if model == "small" else g5_model(32, 320)
    lens = (96, 320, 150, 200, 77, 260)
    log(f"[window batched] {model} {qtile} prompts {lens}")
    W = sw.model_weights(cfg, gain_std=0.1)
    reps = run_e2e_batched(cfg, W, cfg.sampling, 4, list(lens))
    for rep in reps:
        _check(rep, cfg)


@pytest.mark.parametrize("name", ["tiny", "small"])
@pytest.mark.parametrize("mode", ["greedy", "sampled"])
def test_block16_e2e(name, mode):
    """Blocks of 16 positions (15 drafts; the largest block the boundary takes): the fused decode
    attention holds the block's 16 keys in its LDS page, and every other kernel sees 16 rows per
    request."""
    base = synth.TINY if name == "tiny" else small_short()
    cfg = with_block(base, 16)
    log(f"[block 16] {name} {mode}")
    W = sw.model_weights(cfg, gain_std=0.1)
    sp = synth.GREEDY if mode == "greedy" else cfg.sampling
    _, rep, _ = run_e2e(cfg, W, sp, 48 if name == "tiny" else 32)
    _check(rep, cfg)


def test_small_configured_teacher_forced():
    """The small model as configured: a 512-token prompt, 512 generated tokens at T = 1 / top-k 20 /
    top-p 0.95 (Philox seed 1), every step compared with the oracle teacher-forced on the device's
    tokens: logits and draft logits within 2e-2 for the whole run, decisions bit-exact."""
    cfg = synth.SMALL
    log(f"[small as configured] prompt {cfg.prompt_len}, {cfg.gen_len} tokens")
    W = sw.model_weights(cfg, gain_std=0.1)
    stream, rep, _ = run_e2e(cfg, W, cfg.sampling, cfg.gen_len, log_every=64)
    assert len(stream) == cfg.gen_len
    _check(rep, cfg)


def _tau_law(r: float, B: int):
    """Acceptance length under greedy verification when each draft is corrupted independently with
    probability r: tau = j for a first corruption at draft j (j < B), B if none."""
    p = np.array([(1 - r) ** (j - 1) * r for j in range(1, B)] + [(1 - r) ** (B - 1)])
    j = np.arange(1, B + 1)
    mean = float((p * j).sum())
    return mean, float((p * j * j).sum() - mean ** 2)


def test_small_planted_corruption_sweep():
    """The planted drafter on the device at the configured corruption rates r in {0, 0.1, 0.3, 0.6}
    (small model, 512-token prompt, 512 tokens, block 8, greedy verification): every emitted stream
    equals the device's greedy plain-decoding stream G, and the mean acceptance length matches
    E[tau] = (1 - (1 - r)^B) / r (8 / 5.695 / 3.141 / 1.666) within 4.5 standard errors of the
    law's own variance."""
    from synth import gpu as sg
    from speculative_decoding_dflash_amd.runner import Engine
    cfg = synth.SMALL
    t, d = cfg.target, cfg.drafter
    P, B, V, n_gen = cfg.prompt_len, d.block_size, t.vocab, cfg.gen_len
    Wt = sg.model_weights(cfg)
    eng = Engine(cfg, Wt, max_slots=1)
    eng.kv_alloc(0, P + n_gen + 4 * B)
    prompt = torch.from_numpy(sw.prompt_ids(V, d.mask_id, P, 0)).to("cuda")
    g = samp(synth.GREEDY)
    eng.prefill([0], prompt.view(1, -1), [g])
    gen = [int(eng.out[0])]
    while len(gen) < n_gen + B:
        eng.ar_step([0], [g])
        gen.append(int(eng.out[0]))
    G = np.concatenate([prompt.cpu().numpy(), np.array(gen)]).astype(np.int64)
    rows = []
    for r in cfg.corruption_rates:
        eng.prefill([0], prompt.view(1, -1), [g])
        stream, taus, n = [int(eng.out[0])], [], P
        while len(stream) < n_gen:
            pl = sw.planted_drafts(G, n, B - 1, V, d.mask_id, r)
            eng.spec_step([0], [g], planted=torch.from_numpy(pl).to("cuda").view(1, -1))
            tau = int(eng.n_out[0])
            stream.extend(int(x) for x in eng.out[:tau].cpu().numpy())
            taus.append(tau)
            n += tau
        eng.status()
        assert stream[:n_gen] == [int(x) for x in G[P:P + n_gen]], f"rate {r}: stream differs from G"
        closed = B if r == 0 else (1 - (1 - r) ** B) / r
        mean, var = _tau_law(r, B)
        assert abs(mean - closed) < 1e-12
        m = float(np.mean(taus))
        z = 0.0 if var == 0 else (m - closed) / np.sqrt(var / len(taus))
        rows.append((r, len(taus), m, closed, z))
        log(f"  r {r}: {len(taus)} steps, mean tau {m:.3f} vs {closed:.3f} (z {z:.2f})")
        if r == 0:
            assert all(x == B for x in taus)
        assert abs(z) < 4.5
    eng.close()
    del Wt
    torch.cuda.empty_cache()
