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
