"""Host-side arithmetic of bench.py (CPU): the algorithmic step bytes and flops it divides by."""
import math

import numpy as np

import bench
import synth


def _weight_bytes_from_shapes(cfg):
    """Every projection or table read once per step, from the model's tensor list: all weight
    tensors but the embedding table (a step gathers only its block rows), plus the LM head a second
    time (the drafter shares it)."""
    e = 2 if cfg.target.dtype == "bf16" else 4
    n = 0
    for name, shape, kind in synth.tensor_shapes(cfg.target, cfg.drafter):
        if kind == "w" and name != "t.embed":
            n += math.prod(shape)
    n += cfg.target.vocab * cfg.target.hidden
    return n * e


def test_step_bytes_weights_match_tensor_shapes():
    for name in ("27b", "4b", "small"):
        cfg = synth.CONFIGS[name]
        kv_logits = bench._kv_logit_bytes(cfg, 0)
        assert bench.step_bytes(cfg, 0) - kv_logits == _weight_bytes_from_shapes(cfg)


def test_step_bytes_27b_figures():
    cfg = synth.CONFIGS["27b"]
    t, d = cfg.target, cfg.drafter
    # KV read per committed token: 64 layers x K and V x 8 heads x 128 x bf16 = 256 KiB; the drafter's
    # five layers read at most the 2048-token window
    per_tok = bench.step_bytes(cfg, 1001) - bench.step_bytes(cfg, 1000)
    assert per_tok == 256 * 1024 + 20 * 1024
    assert bench.step_bytes(cfg, 5001) - bench.step_bytes(cfg, 5000) == 256 * 1024
    assert 49.2e9 < bench.step_bytes(cfg, 1040) < 49.4e9


def test_batched_bytes_and_flops():
    cfg = synth.CONFIGS["27b"]
    ns = [1024, 2048, 777]
    one = [bench.step_bytes(cfg, n) for n in ns]
    w = bench.step_bytes(cfg, 0) - bench._kv_logit_bytes(cfg, 0)
    assert bench.step_bytes_batch(cfg, ns[:1]) == one[0]
    assert np.isclose(bench.step_bytes_batch(cfg, ns), w + sum(b - w for b in one))
    # flops: the weight term scales with the requests, attention with each request's keys
    f1 = bench.step_flops_batch(cfg, [1024], [1])
    f2 = bench.step_flops_batch(cfg, [1024, 1024], [1, 1])
    assert np.isclose(f2, 2 * f1)
    t = cfg.target
    B, Ld = cfg.drafter.block_size, cfg.drafter.layers
    # one more key per query: QK^T and PV (2 x 2 flops per key and dimension) in every target layer, and
    # in every drafter layer while the context is inside the drafter's 2048-token window
    d_att = bench.step_flops_batch(cfg, [1025], [1]) - f1
    assert np.isclose(d_att, 4.0 * B * t.q_heads * t.head_dim * (t.layers + Ld))
    d_far = bench.step_flops_batch(cfg, [5001], [1]) - bench.step_flops_batch(cfg, [5000], [1])
    assert np.isclose(d_far, 4.0 * B * t.q_heads * t.head_dim * t.layers)


def test_prefill_flops():
    cfg = synth.CONFIGS["27b"]
    t, d = cfg.target, cfg.drafter
    # a prompt of P rows: every projection over P rows (2 flops per multiply-add of the layer's weight
    # matrices), the LM head over one row, causal attention over P (P + 1) / 2 (query, key) pairs, and
    # the injection of the rows the drafter's window can still see (at most W + B of them)
    P = 100
    lp = sum(math.prod(s) for n, s, k in synth.tensor_shapes(t, d) if n.startswith("t.L0.") and k == "w" and len(s) == 2)
    inj = len(d.taps) * t.hidden * t.hidden + d.layers * 2 * t.kv_dim * t.hidden
    want = (2.0 * P * t.layers * lp + 2.0 * t.vocab * t.hidden + 4.0 * t.q_heads * t.head_dim * P * (P + 1) / 2 * t.layers
            + 2.0 * P * inj)
    assert np.isclose(bench.prefill_flops(cfg, [P]), want)
    long_p = 6000  # past the window: the injection is capped at W + B rows
    extra = bench.prefill_flops(cfg, [long_p + 1]) - bench.prefill_flops(cfg, [long_p])
    assert np.isclose(extra, 2.0 * t.layers * lp + 4.0 * t.q_heads * t.head_dim * (long_p + 1) * t.layers)
    assert np.isclose(bench.prefill_flops(cfg, [P, P]), 2 * bench.prefill_flops(cfg, [P]))
