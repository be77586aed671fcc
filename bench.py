#!/usr/bin/env python3
"""Accepted tokens/s of the lossless block speculative-decoding step on one MI355X.

Default workload: the 27B-shaped target (64 layers, hidden 5120, 40 q / 8 kv heads x 128, SwiGLU FFN
17408, vocab 151936, bf16 weights drawn from N(0, 0.02)) with a 5-layer drafter of the same width
(sliding window 2048, taps at target layers 5/19/33/47/61), block size 8, concurrency 1, a 1024-token
prompt of uniform ids, T = 1.0 / top-k 20 / top-p 0.95 with Philox seed 1.  All inputs are synthetic
(the counter-based generator of synth/); nothing is downloaded or read from disk.

Printed, one JSON line: `value` = accepted tokens/s of that run with the real drafter (tokens
emitted per second over the timed steps); with random weights the acceptance length is near 1, so
the same kernels are also run with a planted drafter (drafts taken from the target's greedy stream
and forced to fail at a chosen position, greedy verification) for acceptance lengths 1..8, and as
plain decoding (one target forward per token) for the same-kernel AR baseline, and with stochastic
drafts (drawn from the drafter's own distribution, accepted with min(1, p/q)).  `roofline` reports
the projection kernel (the dominant one: ~99% of the step's bytes): the projection launches of one
step are recorded by the library and replayed back to back between two HIP events on the step's
stream; `traffic` is the HBM bytes per launch measured with rocprofv3 counters.  `cpu_baseline` times
the CPU oracle on a bounded sample.  `batched_configured_runs` adds short configured runs of the same
step over 8 and 32 requests (prompts of 1024 tokens) on the same weights.

--concurrency C and --config 27b-long run the batched measurement alone (with its planted sweep and the
projection replay), printing their own JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from dataclasses import replace

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "accepted tokens/s at conc 1 (27B-shape, block 8); step HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
# HBM bytes per projection launch of the decode step, from rocprofv3 FETCH_SIZE / WRITE_SIZE passes
# scaled by a plain 1 GiB copy (profiles/gemm_kernel_27b_conc1_traffic.txt), and the hash of the
# kernel source they were taken on: a changed kernel reports null until the counters are retaken.
GEMM_TRAFFIC = {"bytes_per_launch": 177535881, "gemm_src_sha256_16": "b7e9ec76474e2219"}


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def step_bytes(cfg, n: int) -> float:
    """Algorithmic HBM bytes of one draft + verify + accept step starting at committed length n:
    every weight once (the drafter re-reads the shared LM head), the KV read by both attentions,
    the KV written for the block, and the fp32 logits written and read."""
    t, d = cfg.target, cfg.drafter
    e = 2 if t.dtype == "bf16" else 4
    B = d.block_size
    layer = t.layer_params()
    target_w = (t.layers * layer + t.vocab * t.hidden) * e
    drafter_w = (d.layers * layer + len(d.taps) * t.hidden * t.hidden + t.vocab * t.hidden) * e
    kv_t = t.layers * 2 * t.kv_dim * e  # per token
    kv_d = d.layers * 2 * t.kv_dim * e
    keys_t = n + B
    keys_d = (min(n, d.window) if d.window else n) + B
    kv = keys_t * kv_t + keys_d * kv_d + B * (kv_t + kv_d)
    logits = 2 * 4 * (2 * B - 1) * t.vocab
    return float(target_w + drafter_w + kv + logits)


def ar_bytes(cfg, n: int) -> float:
    t = cfg.target
    e = 2 if t.dtype == "bf16" else 4
    return float((t.layers * t.layer_params() + t.vocab * t.hidden) * e + (n + 1) * t.layers * 2 * t.kv_dim * e
                 + 2 * 4 * t.vocab)


class Timer:
    def __init__(self, torch):
        self.torch = torch
        self.e0 = torch.cuda.Event(enable_timing=True)
        self.e1 = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.torch.cuda.synchronize()
        self.e0.record()

    def stop(self) -> float:
        self.e1.record()
        self.torch.cuda.synchronize()
        return self.e0.elapsed_time(self.e1)


def run_spec(eng, torch, prompt, samp, warmup, steps, planted=None, profile=False, graph=True, stochastic=False):
    """Prefill, then warmup + timed speculative steps with no host synchronisation inside the timed
    region (device-resident sequence state).  With graph=True the step is captured once into a HIP
    graph after the warmup and replayed (every launch parameter of a step is fixed on the host);
    planted drafts are then copied into the captured buffer before each replay.  Returns (ms for the
    timed steps, taus per step); with profile=True (eager steps) the library records the projection
    launches of the timed steps.  stochastic: drafts drawn from the drafter's own distributions."""
    from speculative_decoding_dflash_amd import binding as Bd
    taus = torch.zeros(warmup + steps, dtype=torch.int32, device="cuda")
    eng.prefill([0], prompt.view(1, -1), [samp])
    use_graph = graph and not profile
    # with a graph, its first launch is the last warmup step; it is captured after at least one eager step,
    # so that its launches have the decode shapes (right after a prefill the drafter's injection covers
    # every prompt row)
    n_eager = max(1, warmup - 1) if use_graph else warmup
    for i in range(n_eager):
        eng.spec_step([0], [samp], planted=None if planted is None else planted[i], stochastic=stochastic)
        taus[i:i + 1].copy_(eng.n_out[:1])
    g = pl = None
    if use_graph:
        pl = None if planted is None else planted[0].clone()
        g = eng.capture_spec_step([0], [samp], planted=pl, stochastic=stochastic)
        if n_eager < warmup:
            if pl is not None:
                pl.copy_(planted[n_eager])
            g.replay()
            taus[n_eager:n_eager + 1].copy_(eng.n_out[:1])
    tm = Timer(torch)
    tm.start()
    if profile:
        Bd.dflash_profile(eng.ctx, True)
    for i in range(warmup, warmup + steps):
        if g is not None:
            if pl is not None:
                pl.copy_(planted[i])
            g.replay()
        else:
            eng.spec_step([0], [samp], planted=None if planted is None else planted[i], stochastic=stochastic)
        taus[i:i + 1].copy_(eng.n_out[:1])
    ms = tm.stop()
    eng.status()
    return ms, [int(x) for x in taus.cpu().tolist()]


def step_bytes_batch(cfg, ns) -> float:
    """step_bytes for a batch of requests at committed lengths ns: the weights are read once per step
    whatever the batch, the KV and logits terms once per request."""
    one_req = [step_bytes(cfg, n) for n in ns]
    w = step_bytes(cfg, 0) - _kv_logit_bytes(cfg, 0)
    return float(w + sum(b - w for b in one_req))


def _kv_logit_bytes(cfg, n: int) -> float:
    t, d = cfg.target, cfg.drafter
    e = 2 if t.dtype == "bf16" else 4
    B = d.block_size
    kv_t, kv_d = t.layers * 2 * t.kv_dim * e, d.layers * 2 * t.kv_dim * e
    keys_d = (min(n, d.window) if d.window else n) + B
    return float((n + B) * kv_t + keys_d * kv_d + B * (kv_t + kv_d) + 2 * 4 * (2 * B - 1) * t.vocab)


def step_flops_batch(cfg, ns, taus) -> float:
    """Algorithmic flops of one batched step: 2 per multiply-add of every projection over the rows
    that pass through it (block rows through both models, the drafter's LM head on B-1 rows, the
    injection over the rows committed by the previous step) plus both attentions (QK^T and PV over
    every key a query sees)."""
    t, d = cfg.target, cfg.drafter
    B, H, V = d.block_size, t.hidden, t.vocab
    c = len(ns)
    lp = t.layer_params()
    f = 2.0 * c * B * (t.layers * lp + V * H)                      # verify + target LM head
    f += 2.0 * c * B * d.layers * lp + 2.0 * c * (B - 1) * V * H   # drafter block forward + shared LM head
    f += 2.0 * sum(taus) * (len(d.taps) * H * H + d.layers * 2 * t.kv_dim * H)  # injection
    for n in ns:
        f += 4.0 * B * t.q_heads * t.head_dim * (n + B) * t.layers
        f += 4.0 * B * t.q_heads * t.head_dim * ((min(n, d.window) if d.window else n) + B) * d.layers
    return f


def prefill_flops(cfg, lens) -> float:
    """Algorithmic flops of prefilling prompts of the given lengths (one verify over every prompt row and
    the drafter injection of the rows a sliding window can still see): 2 per multiply-add of every
    projection over its rows (the LM head over one logits row per prompt), plus causal attention (QK^T
    and PV over keys 0..p for the query at p)."""
    t, d = cfg.target, cfg.drafter
    H, V = t.hidden, t.vocab
    lp = t.layer_params()
    f = 0.0
    for P in lens:
        f += 2.0 * P * t.layers * lp + 2.0 * V * H
        f += 4.0 * t.q_heads * t.head_dim * (P * (P + 1) / 2) * t.layers
        inj = min(P, d.window + d.block_size) if d.window else P
        f += 2.0 * inj * (len(d.taps) * H * H + d.layers * 2 * t.kv_dim * H)
    return f


def cpu_baseline(cfg, tau: float):
    """The oracle (float64 numpy, as it stands) on a bounded sample of one step of the workload: one
    27B-shaped target layer over a block of 8 at context 1536 (random cache contents), the LM head over
    a 1/16 slice of the vocabulary and the drafter's fc projection, each run repeatedly for a few seconds
    and averaged, then scaled by layer and vocabulary counts to one draft + verify step."""
    import numpy as np
    import synth
    from oracle import ops
    from oracle.model import Target
    from synth import weights as sw
    threads = len(os.sched_getaffinity(0))
    t, d = cfg.target, cfg.drafter
    B, ctx = d.block_size, 1536
    vs = t.vocab // 16
    one = replace(cfg, target=replace(t, layers=1, vocab=vs), drafter=replace(d, taps=(0,), layers=1))
    names = [n for n, _, _ in synth.tensor_shapes(one.target, one.drafter) if n.startswith("t.")]
    W = sw.model_weights(one, names=names)
    tg = Target(one.target, W, taps=())
    cache = tg.new_cache()
    cache.ensure(ctx + B)
    rng = np.random.default_rng(0)
    cache.k[0][:ctx] = rng.standard_normal(cache.k[0][:ctx].shape)
    cache.v[0][:ctx] = rng.standard_normal(cache.v[0][:ctx].shape)
    toks = list(range(B))

    def timed(fn, budget_s: float):
        """Mean wall time of fn over repeated calls until about budget_s seconds have run (at least 2)."""
        n, t0 = 0, time.perf_counter()
        while True:
            fn()
            n += 1
            el = time.perf_counter() - t0
            if n >= 2 and el >= budget_s:
                return el / n, n

    # the one-layer forward (its LM head over the vocabulary slice included), the slice alone, the fc
    t_fwd, n_fwd = timed(lambda: tg.forward(cache, toks, ctx, logit_rows=B), 8.0)
    x = rng.standard_normal((B, t.hidden))
    t_lm, n_lm = timed(lambda: ops.linear(x, tg.w["t.lm_head"]), 2.0)
    fc = sw.tensor("d.fc", (t.hidden, len(d.taps) * t.hidden), "w", cfg.weight_seed, cfg.weight_std, t.dtype)
    fc = fc.astype(np.float64)
    xf = rng.standard_normal((B, len(d.taps) * t.hidden))
    t_fc, n_fc = timed(lambda: ops.linear(xf, fc), 2.0)
    t_layer = max(t_fwd - t_lm, 1e-9)
    lm_full = t_lm * t.vocab / vs
    step_s = (t.layers + d.layers) * t_layer + t_fc + lm_full * (1 + (B - 1) / B)
    return {"value": round(tau / step_s, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "step_s": round(step_s, 3),
            "sample": f"oracle (float64 numpy) timed on one target layer over a block of {B} at context {ctx} "
                      f"({n_fwd} runs), the LM head over {vs} of {t.vocab} vocabulary rows ({n_lm} runs) and the "
                      f"drafter fc ({n_fc} runs), means over ~12 s of CPU work; scaled to {t.layers}+{d.layers} "
                      f"layers and the full vocabulary; accepted tokens/s at the GPU run's tau {tau:.3f}"}


MFMA_PEAK_TFS = 2500.0  # dense bf16 MFMA, MI355X published
SETTLE_STEPS = 32  # untimed launches of a throwaway graph before the first timed leg


def batch_main(args, cfg, conc: int, weights=None, quick: bool = False):
    """Batched steps: `conc` requests decoded together (each step verifies conc x B rows and drafts
    conc blocks).  Requests are prefilled one by one (prompt lengths from the workload: fixed, or
    uniform over the long-context range), their prompts injected into the drafter, then every timed
    step is one captured HIP graph of verify -> accept -> draft over all requests.  Printed: one JSON
    line with accepted tokens/s of the configured run (T=1 / top-k / top-p, real drafter) and a
    planted sweep under greedy verification (every request forced to acceptance length tau*), each
    with the step's algorithmic HBM and MFMA fractions.  quick: the configured run only, on the
    given weights, returned as a dict instead of printed."""
    import numpy as np
    import torch

    from synth import gpu as sgpu
    from synth import weights as sw
    from speculative_decoding_dflash_amd import binding as Bd
    from speculative_decoding_dflash_amd.runner import Engine, sampling

    t, d = cfg.target, cfg.drafter
    B, V = d.block_size, t.vocab
    K, Wm = args.steps, args.warmup
    if cfg.prompt_len_range:
        lens = [int(x) for x in sw.prompt_lengths(cfg.prompt_len_range[0], cfg.prompt_len_range[1], conc, 0)]
    else:
        lens = [cfg.prompt_len] * conc
    taus_sweep = [int(x) for x in args.tau_sweep.split(",")] if args.tau_sweep else list(range(1, B + 1))
    log(f"[bench] {cfg.name}, concurrency {conc}, prompt lengths {min(lens)}..{max(lens)} "
        f"(mean {sum(lens) / conc:.0f})")
    if weights is None:
        log("[bench] generating weights on the GPU")
        weights = sgpu.model_weights(cfg)
        torch.cuda.synchronize()
    n_ar = (Wm + K + 1) * B + 2 * B  # greedy tokens needed per request by the planted sweep
    max_tokens = max(lens) + max(n_ar, (Wm + K + 2) * B) + 2 * B
    eng = Engine(cfg, weights, max_slots=conc, max_rows=max(max(lens), conc * B),
                 max_pages_per_seq=max_tokens // 16 + 4)
    slots = list(range(conc))
    for r in slots:
        eng.kv_alloc(r, max_tokens)
    prompts = [torch.from_numpy(sw.prompt_ids(V, d.mask_id, lens[r], r)).to("cuda") for r in slots]
    sp = cfg.sampling
    s_conf = sampling(sp.temperature, sp.top_k, sp.top_p, sp.seed)
    s_greedy = sampling(0.0, 0, 1.0, 1)

    def prefill_all(samp, inject=True):
        """Prefill every request; returns (seconds, first tokens [conc] on the device)."""
        first = torch.zeros(conc, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        t0 = time.time()
        for r in slots:
            eng.prefill([r], prompts[r].view(1, -1), [samp])
            first[r:r + 1].copy_(eng.out[:1])
            if inject:  # the prompt's features go into the drafter cache before the next prefill
                Bd.dflash_draft_block(eng.ctx, [r], eng.feats, eng.block[r * B:], None)
        torch.cuda.synchronize()
        return time.time() - t0, first

    def step(samp, pl=None):
        eng.verify(slots, eng.block, B, False, B)
        eng.accept(slots, B - 1, [samp] * conc)
        eng.draft(slots)
        if pl is not None:
            eng.block.view(-1, B)[:conc, 1:] = pl

    def run(samp, planted=None):
        """Prefill, warmup steps, then K timed replays of the captured step; returns (ms, taus [steps][conc],
        committed lengths at the start of every timed step)."""
        sec, _ = prefill_all(samp)
        if planted is not None:
            eng.block.view(-1, B)[:conc, 1:] = planted[0]
        taus = torch.zeros(Wm + K, conc, dtype=torch.int32, device="cuda")
        # the graph's first launch is the last warmup step; captured after at least one eager step
        n_eager = Wm - 1 if Wm > 1 else Wm
        for i in range(n_eager):
            step(samp, None if planted is None else planted[i + 1])
            taus[i].copy_(eng.n_out[:conc])
        pl = None if planted is None else planted[n_eager + 1].clone()
        if getattr(args, "no_graph", False):  # counter runs: every step issued eagerly
            for i in range(n_eager, Wm):
                step(samp, None if planted is None else planted[i + 1])
                taus[i].copy_(eng.n_out[:conc])
            tm = Timer(torch)
            tm.start()
            for i in range(Wm, Wm + K):
                step(samp, None if planted is None else planted[i + 1])
                taus[i].copy_(eng.n_out[:conc])
            ms = tm.stop()
            eng.status()
            tl = taus.cpu().numpy()
            ns = [[lens[r] + int(tl[:i, r].sum()) for r in slots] for i in range(Wm, Wm + K)]
            return ms, tl[Wm:], ns, sec
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(samp, pl)
        if n_eager < Wm:
            if pl is not None:
                pl.copy_(planted[n_eager + 1])
            g.replay()
            taus[n_eager].copy_(eng.n_out[:conc])
        tm = Timer(torch)
        tm.start()
        for i in range(Wm, Wm + K):
            if pl is not None:
                pl.copy_(planted[i + 1])
            g.replay()
            taus[i].copy_(eng.n_out[:conc])
        ms = tm.stop()
        eng.status()
        tl = taus.cpu().numpy()
        ns = [[lens[r] + int(tl[:i, r].sum()) for r in slots] for i in range(Wm, Wm + K)]
        return ms, tl[Wm:], ns, sec

    def summary(ms, tl, ns):
        tok = int(tl.sum())
        byt = sum(step_bytes_batch(cfg, n) for n in ns) / K
        # the injection of step i covers the rows committed by step i-1
        fl = sum(step_flops_batch(cfg, ns[i], tl[i - 1] if i > 0 else tl[0]) for i in range(K)) / K
        mss = ms / K
        return {"tok_s": round(tok / (ms / 1e3), 1), "ms_per_step": round(mss, 3),
                "tau": round(tok / (K * conc), 4),
                "step_hbm_gbs": round(byt / (mss / 1e3) / 1e9, 1),
                "step_hbm_frac": round(byt / (mss / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                "step_tflops": round(fl / (mss / 1e3) / 1e12, 1),
                "step_mfma_frac": round(fl / (mss / 1e3) / 1e12 / MFMA_PEAK_TFS, 4),
                "step_bytes": byt, "step_flops": fl}

    if not quick:  # a throwaway graph launched before the first timed leg (see SETTLE_STEPS)
        log(f"[bench] settle: untimed graph launches")
        prefill_all(s_conf)
        step(s_conf)  # captured after a step, like the timed legs' graphs
        g_settle = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_settle):
            step(s_conf)
        for _ in range(min(SETTLE_STEPS, (max_tokens - max(lens)) // B - 3)):
            g_settle.replay()
        torch.cuda.synchronize()
        del g_settle
    log(f"[bench] configured run: {Wm} warmup + {K} timed steps")
    ms, tl, ns, pre_s = run(s_conf)
    conf = summary(ms, tl, ns)
    log(f"[bench]   {conf} (prefill of all requests {pre_s:.1f} s)")
    if quick:
        eng.close()
        return {k: v for k, v in conf.items() if k not in ("step_bytes", "step_flops")} | {
            "step_gbytes": round(conf["step_bytes"] / 1e9, 2), "step_tflop": round(conf["step_flops"] / 1e12, 3),
            "prompt_len": lens[0], "steps": K, "warmup": Wm}

    # projection roofline at this batch: the projection launches of one eager step, replayed
    prefill_all(s_conf)
    Bd.dflash_profile(eng.ctx, True)
    step(s_conf)
    Bd.dflash_profile(eng.ctx, False)
    torch.cuda.synchronize()
    reps = args.profile_steps
    rep_ms, rep_bytes, rep_n = Bd.dflash_profile_replay(eng.ctx, reps)
    gemm_ms = rep_ms / reps
    rows_proj = conc * B
    log(f"[bench] projections: {rep_n} launches per step, {gemm_ms:.3f} ms replayed back to back, "
        f"{rep_bytes / (gemm_ms / 1e3) / 1e9:.0f} GB/s")

    sweep = {}
    if not args.no_sweep:
        # The greedy stream of every request, emitted by greedy speculative decoding over the same batch:
        # a verify row's logits depend only on its prefix, so the planted runs below (same kernels, same
        # batch) reproduce it exactly, where plain decoding (other row tiles, other fp32 summation
        # orders) may part from it at a near tie.
        log(f"[bench] greedy stream for the planted drafter: {n_ar} tokens per request")
        _, first = prefill_all(s_greedy)
        gen = [[int(x)] for x in first.cpu().tolist()]
        while min(len(x) for x in gen) < n_ar:
            step(s_greedy)
            taus = eng.n_out[:conc].cpu().tolist()
            outs = eng.out[:conc * B].view(conc, B).cpu().numpy()
            for r in slots:
                gen[r].extend(int(x) for x in outs[r, :taus[r]])
        eng.status()
        G = [np.concatenate([prompts[r].cpu().numpy(), np.array(gen[r][:n_ar])]).astype(np.int64) for r in slots]
        for ts in taus_sweep:
            plans = []
            for i in range(Wm + K + 1):
                plans.append(np.stack([sw.planted_drafts(G[r], lens[r] + ts * i, B - 1, V, d.mask_id, 0.0,
                                                         force_reject_at=ts if ts < B else None) for r in slots]))
            planted = torch.from_numpy(np.stack(plans)).to("cuda")
            ms_p, tl_p, ns_p, _ = run(s_greedy, planted)
            assert (tl_p == ts).all(), (ts, tl_p)
            sweep[str(ts)] = {k: v for k, v in summary(ms_p, tl_p, ns_p).items() if k not in ("step_bytes", "step_flops")}
            log(f"[bench]   planted tau*={ts}: {sweep[str(ts)]}")

    out = {
        "metric": f"accepted tokens/s at conc {conc} ({cfg.name}-shape, block {B}); step HBM and MFMA fractions",
        "value": conf["tok_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": conf["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if t.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}-shaped target ({t.layers} layers, hidden {t.hidden}, {t.q_heads}q/{t.kv_heads}kv x "
                        f"{t.head_dim}, FFN {t.ffn}, vocab {t.vocab}) + {d.layers}-layer drafter (window {d.window}, "
                        f"taps {list(d.taps)}); block {B}, concurrency {conc}, prompts of "
                        + (f"{min(lens)}..{max(lens)} (uniform over {cfg.prompt_len_range}, mean "
                           f"{sum(lens) / conc:.0f})" if cfg.prompt_len_range else f"{lens[0]}")
                        + f" uniform ids, T={sp.temperature}/top-k {sp.top_k}/top-p {sp.top_p}, Philox seed {sp.seed}",
            "block": B, "concurrency": conc, "prompt_lens": [min(lens), max(lens), round(sum(lens) / conc, 1)],
        },
        "configured": conf,
        "prefill_s": round(pre_s, 2),
        "prefill_tok_s": round(sum(lens) / pre_s, 1),
        "prefill": {"requests": conc, "tokens": int(sum(lens)), "s": round(pre_s, 3),
                    "tok_s": round(sum(lens) / pre_s, 1), "tflop": round(prefill_flops(cfg, lens) / 1e12, 2),
                    "tflops": round(prefill_flops(cfg, lens) / pre_s / 1e12, 1),
                    "mfma_frac": round(prefill_flops(cfg, lens) / pre_s / 1e12 / MFMA_PEAK_TFS, 4),
                    "method": "each request prefilled in turn (one verify over its prompt rows, then the "
                              "drafter injection), wall clock with a device synchronisation at both ends"},
        "tau_sweep_planted_greedy": sweep,
        "projections": {"launches_per_step": rep_n, "ms_per_step": round(gemm_ms, 4), "rows": rows_proj,
                        "hbm_gbs": round(rep_bytes / (gemm_ms / 1e3) / 1e9, 1),
                        "hbm_frac": round(rep_bytes / (gemm_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                        "method": "the projection launches of one eager step recorded by the library and replayed "
                                  f"{reps} times back to back between two HIP events on the step's stream"},
    }
    print(json.dumps(out), flush=True)
    eng.close()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--config", default="27b")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-ar", action="store_true", help="skip plain decoding (and so the planted sweep)")
    ap.add_argument("--profile-steps", type=int, default=8, help="replay passes for the projection roofline")
    ap.add_argument("--no-graph", action="store_true", help="issue every timed step eagerly instead of replaying "
                                                            "a captured HIP graph of the step")
    ap.add_argument("--concurrency", type=int, default=None,
                    help="requests decoded together (default: the workload's own, 1 for 27b); above 1 the "
                         "batched measurement runs instead of the concurrency-1 line")
    ap.add_argument("--tau-sweep", default="", help="planted acceptance lengths of the batched sweep, e.g. 1,3,5,7")
    ap.add_argument("--no-batched", action="store_true",
                    help="skip the short configured runs at concurrency 8 and 32 appended to the default line")
    ap.add_argument("--block", type=int, default=None,
                    help="block size (1 anchor + block-1 drafts) instead of the configuration's own")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="first copy 1 GiB device to device (a plain copy of known size, the reference for "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.block is not None and not 2 <= args.block <= 16:
        print("--block takes 2 .. 16", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): this build measures the "
              "single-GPU step; the path would shard by request, see the design notes.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from synth import gpu as sgpu
    from synth import weights as sw
    from speculative_decoding_dflash_amd import binding as Bd
    from speculative_decoding_dflash_amd.runner import Engine, sampling

    cfg = synth.CONFIGS[args.config]
    if args.block is not None:
        from dataclasses import replace
        cfg = replace(cfg, drafter=replace(cfg.drafter, block_size=args.block))
    conc = args.concurrency or cfg.concurrency
    if conc > 1 or cfg.prompt_len_range:
        batch_main(args, cfg, conc)
        return
    t, d = cfg.target, cfg.drafter
    B, P, V = d.block_size, cfg.prompt_len, t.vocab
    K, Wm = args.steps, args.warmup
    if args.calibration_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 1 GiB read, 1 GiB written")
        del src, dst
    log(f"[bench] {cfg.name}: generating weights on the GPU")
    t0 = time.time()
    weights = sgpu.model_weights(cfg)
    torch.cuda.synchronize()
    log(f"[bench] weights ready in {time.time() - t0:.1f}s "
        f"({sum(w.numel() * w.element_size() for w in weights.values()) / 1e9:.2f} GB)")
    settle = 0 if args.no_graph else SETTLE_STEPS  # the settle phase exists for graph launches
    max_tokens = P + (max(Wm + K, settle + 1) + 2) * B + 2 * B
    eng = Engine(cfg, weights, max_slots=1, max_rows=P, max_pages_per_seq=max_tokens // 16 + 4)
    eng.kv_alloc(0, max_tokens)
    prompt = torch.from_numpy(sw.prompt_ids(V, d.mask_id, P, 0)).to("cuda")
    sp = cfg.sampling
    s_conf = sampling(sp.temperature, sp.top_k, sp.top_p, sp.seed)
    s_greedy = sampling(0.0, 0, 1.0, 1)

    # untimed settle phase: the first ~24 launches of the first captured graph of a process have run ~3%
    # slower on this part (per-step events: 11.2 ms, then 10.8 ms; graphs captured later run at full
    # speed from their first launch), so a throwaway graph is launched `settle` times before any timed leg
    if settle:
        log(f"[bench] settle: {settle} untimed graph launches")
        eng.prefill([0], prompt.view(1, -1), [s_conf])
        eng.spec_step([0], [s_conf])  # captured after a step, like the timed legs' graphs
        g_settle = eng.capture_spec_step([0], [s_conf])
        for _ in range(settle):
            g_settle.replay()
        torch.cuda.synchronize()
        del g_settle

    # 1. the configured run: real drafter, T=1 / top-k / top-p
    log(f"[bench] configured run: {Wm} warmup + {K} timed steps")
    graph = not args.no_graph
    ms, taus = run_spec(eng, torch, prompt, s_conf, Wm, K, graph=graph)
    tk = taus[Wm:]
    tau = sum(tk) / K
    ms_step = ms / K
    tok_s = sum(tk) / (ms / 1e3)
    n0 = P + sum(taus[:Wm])
    ns = [n0 + sum(tk[:i]) for i in range(K)]
    bytes_step = sum(step_bytes(cfg, n) for n in ns) / K
    log(f"[bench]   tau {tau:.3f}, {ms_step:.3f} ms/step, {tok_s:.1f} tok/s, "
        f"{bytes_step / ms_step / 1e6:.0f} GB/s algorithmic")

    # 1b. the same configuration with stochastic drafts (each draft drawn from the drafter's own
    #     filtered distribution, accepted with min(1, p/q))
    stoch = None
    if not d.selector_top_k:  # the DFlash2 selector proposes one deterministic path
        ms_q, taus_q = run_spec(eng, torch, prompt, s_conf, Wm, K, graph=graph, stochastic=True)
        tq = taus_q[Wm:]
        stoch = {"tok_s": round(sum(tq) / (ms_q / 1e3), 2), "ms_per_step": round(ms_q / K, 4),
                 "tau": round(sum(tq) / K, 4)}
        log(f"[bench]   stochastic drafts: {stoch}")

    # 2. roofline of the projection kernel: record the projection launches of one decode step, then
    #    replay exactly those launches back to back under one pair of HIP events on the step's stream
    run_spec(eng, torch, prompt, s_conf, 1, 1, profile=True)
    Bd.dflash_profile(eng.ctx, False)
    reps = args.profile_steps
    rep_ms, rep_bytes, rep_n = Bd.dflash_profile_replay(eng.ctx, reps)
    gemm_step_ms = rep_ms / reps
    achieved = rep_bytes / (gemm_step_ms / 1e3) / 1e9
    log(f"[bench] projection kernel: {rep_n} launches per step, {gemm_step_ms:.3f} ms per step's launches "
        f"replayed back to back ({reps} passes), {achieved:.0f} GB/s")

    # 3. same-kernel plain decoding (also the greedy stream for the planted drafter)
    ar = None
    sweep = {}
    if not args.no_ar:
        n_ar_needed = (Wm + K + 1) * B + 2 * B
        log(f"[bench] plain decoding: {n_ar_needed} greedy tokens")
        eng.prefill([0], prompt.view(1, -1), [s_greedy])
        gen = [eng.out[:1].clone()]
        ar_t = Timer(torch)
        ar_timed = min(K * 2, n_ar_needed - 1)
        for i in range(n_ar_needed - 1):
            if i == n_ar_needed - 1 - ar_timed:
                ar_t.start()
            eng.ar_step([0], [s_greedy])
            gen.append(eng.out[:1].clone())
        ar_ms = ar_t.stop()
        eng.status()
        G = np.concatenate([prompt.cpu().numpy(), torch.cat(gen).cpu().numpy()]).astype(np.int64)
        n_ar = P + n_ar_needed - ar_timed
        ar_gbs = sum(ar_bytes(cfg, n_ar + i) for i in range(ar_timed)) / (ar_ms / 1e3) / 1e9
        ar = {"tok_s": round(ar_timed / (ar_ms / 1e3), 2), "ms_per_token": round(ar_ms / ar_timed, 4),
              "hbm_gbs": round(ar_gbs, 1)}
        log(f"[bench]   {ar}")

        # 4. planted drafter, greedy verification, forced acceptance length tau* = 1 .. B
        if not args.no_sweep:
            for ts in range(1, B + 1):
                plans, n = [], P
                for i in range(Wm + K):
                    plans.append(sw.planted_drafts(G, n, B - 1, V, d.mask_id, 0.0,
                                                   force_reject_at=ts if ts < B else None))
                    n += ts
                planted = torch.from_numpy(np.stack(plans)).to("cuda")
                ms_p, taus_p = run_spec(eng, torch, prompt, s_greedy, Wm, K, planted=planted, graph=graph)
                assert all(x == ts for x in taus_p), (ts, taus_p)
                nsw = [P + ts * (Wm + i) for i in range(K)]
                gbs = sum(step_bytes(cfg, x) for x in nsw) / (ms_p / 1e3) / 1e9
                sweep[str(ts)] = {"tok_s": round(ts * K / (ms_p / 1e3), 1), "ms_per_step": round(ms_p / K, 3),
                                  "step_hbm_gbs": round(gbs, 1)}
                log(f"[bench]   planted tau*={ts}: {sweep[str(ts)]}")

    # streaming probe on the same box: a 1 GiB device-to-device copy (torch's copy kernel; 1 GiB read
    # and 1 GiB written), best of 5, for context next to the 8 TB/s published peak
    src = torch.empty(1 << 29, dtype=torch.float16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    best = None
    for _ in range(5):
        pt = Timer(torch)
        pt.start()
        dst.copy_(src)
        t_ms = pt.stop()
        best = t_ms if best is None else min(best, t_ms)
    probe = {"kind": "device-to-device copy, 1 GiB read + 1 GiB written, best of 5",
             "gbs": round(2 * (1 << 30) / (best / 1e3) / 1e9, 1)}
    log(f"[bench] copy probe: {probe['gbs']} GB/s (read + write)")
    del src, dst

    # short configured runs of the same step over batches of requests (the batched path's kernels:
    # all rows of a projection in one tiled launch, batch-aware attention splits), on the same weights
    batched = None
    if not args.no_batched and args.config == "27b" and B == 8:
        eng.close()
        qa = argparse.Namespace(**{**vars(args), "steps": min(K, 8), "warmup": min(Wm, 2)})
        batched = {str(c): batch_main(qa, cfg, c, weights=weights, quick=True) for c in (8, 32)}

    cpu = None
    if not args.no_cpu:
        log("[bench] CPU oracle baseline (bounded sample)")
        cpu = cpu_baseline(cfg, tau)
        log(f"[bench]   {cpu}")

    step_gbs = bytes_step / (ms_step / 1e3) / 1e9
    import hashlib
    src = os.path.join(ROOT, "speculative_decoding_dflash_amd", "csrc", "gemm.hip")
    traffic = GEMM_TRAFFIC["bytes_per_launch"] if args.config == "27b" and B == 8 and hashlib.sha256(
        open(src, "rb").read()).hexdigest()[:16] == GEMM_TRAFFIC["gemm_src_sha256_16"] else None
    out = {
        "metric": METRIC if (cfg.name, B) == ("27b", 8) else
                  f"accepted tokens/s at conc 1 ({cfg.name}-shape, block {B}); step HBM GB/s vs peak",
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if t.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}-shaped target ({t.layers} layers, hidden {t.hidden}, {t.q_heads}q/{t.kv_heads}kv x "
                        f"{t.head_dim}, FFN {t.ffn}, vocab {t.vocab}) + {d.layers}-layer drafter (window {d.window}, "
                        f"taps {list(d.taps)}); block {B}, concurrency 1, prompt {P} uniform ids, "
                        f"T={sp.temperature}/top-k {sp.top_k}/top-p {sp.top_p}, Philox seed {sp.seed}",
            "block": B, "concurrency": 1, "prompt_len": P,
        },
        "tau": round(tau, 4),
        "step_launch": "one captured HIP graph per step, replayed" if graph else "eager launches",
        "step_hbm_gbs": round(step_gbs, 1),
        "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "step_bytes": bytes_step,
        "ar_baseline": ar,
        "tau_sweep_planted_greedy": sweep,
        "stochastic_drafts": stoch,
        "roofline": {"bound": "hbm", "kernel": "gemm_kernel + gemm_sk_kernel (all projections of the step)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0, "
                                     "factors from a 1 GiB copy)",
                     "traffic_vs_algorithmic": None if traffic is None else round(
                         traffic / (rep_bytes / max(rep_n, 1)), 4),
                     "launches_per_step": rep_n, "bytes_per_launch": rep_bytes / max(rep_n, 1),
                     "avg_launch_us": round(gemm_step_ms * 1e3 / max(rep_n, 1), 3),
                     "method": "the projection launches of one decode step recorded by the library and replayed "
                               f"{reps} times back to back between two HIP events on the step's stream"},
        "cpu_baseline": cpu,
        "batched_configured_runs": batched,
        "hbm_copy_probe": probe,
    }
    print(json.dumps(out), flush=True)
    eng.close()


if __name__ == "__main__":
    main()
