"""Pins of the oracle's elementary operations against library routines and invariants."""
import numpy as np
import pytest
import torch

from oracle import ops

RNG = np.random.default_rng(1234)


def test_rms_norm_matches_torch():
    x = RNG.standard_normal((7, 96))
    g = RNG.standard_normal(96)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), weight=torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(ops.rms_norm(x, g, 1e-6), ref, rtol=1e-12, atol=1e-14)


def test_silu_matches_torch():
    x = RNG.standard_normal(1000) * 5
    np.testing.assert_allclose(ops.silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(), rtol=1e-12)


def test_rope_two_dim_rotation_by_hand():
    # d = 2: one pair rotated by angle pos * theta^0 = pos.
    for pos in (0, 1, 5, 37):
        y = ops.rope(np.array([[1.0, 0.0]]), np.array(pos), 1e4)
        np.testing.assert_allclose(y[0], [np.cos(pos), np.sin(pos)], atol=1e-14)
    # d = 4: second pair (indices 1 and 3) turns at theta^(-1/2) per position.
    theta = 100.0
    y = ops.rope(np.array([[0.0, 1.0, 0.0, 0.0]]), np.array(3), theta)
    a = 3 * theta ** -0.5
    np.testing.assert_allclose(y[0], [0.0, np.cos(a), 0.0, np.sin(a)], atol=1e-14)


def test_rope_preserves_norm_and_is_relative():
    d = 64
    q = RNG.standard_normal((1, d))
    k = RNG.standard_normal((1, d))
    for p in (0, 3, 1000):
        np.testing.assert_allclose(np.linalg.norm(ops.rope(q, np.array(p), 1e6)), np.linalg.norm(q), rtol=1e-12)
    dots = [float(ops.rope(q, np.array(m), 1e4)[0] @ ops.rope(k, np.array(m - 5), 1e4)[0]) for m in (5, 17, 900)]
    np.testing.assert_allclose(dots, dots[0], rtol=1e-9)
    # and it is not trivially constant in the offset
    other = float(ops.rope(q, np.array(20), 1e4)[0] @ ops.rope(k, np.array(0), 1e4)[0])
    assert abs(other - dots[0]) > 1e-6


def test_rope_pairs_are_half_split_not_interleaved():
    # rotate-half pairs element i with element i + d/2
    d = 8
    x = np.zeros((1, d))
    x[0, 0] = 1.0
    y = ops.rope(x, np.array(1), 1e4)
    assert abs(y[0, 4] - np.sin(1.0)) < 1e-14 and abs(y[0, 1]) < 1e-14


@pytest.mark.parametrize("hq,hkv", [(4, 4), (6, 2), (5, 1)])
@pytest.mark.parametrize("mask_kind", ["causal", "all", "window"])
def test_attention_matches_sdpa(hq, hkv, mask_kind):
    d, n = 16, 23
    q = RNG.standard_normal((hq, d))
    k = RNG.standard_normal((n, hkv, d))
    v = RNG.standard_normal((n, hkv, d))
    p = 17
    keys = np.arange(n)
    if mask_kind == "causal":
        allowed = keys <= p
    elif mask_kind == "all":
        allowed = np.ones(n, dtype=bool)
    else:
        allowed = (keys >= 19) | ((keys < 19) & (p - keys < 6))
    out = ops.attention(q, k, v, allowed)
    group = hq // hkv
    kt = torch.from_numpy(np.repeat(k, group, axis=1).transpose(1, 0, 2).copy())
    vt = torch.from_numpy(np.repeat(v, group, axis=1).transpose(1, 0, 2).copy())
    qt = torch.from_numpy(q[:, None, :].copy())
    m = torch.from_numpy(np.broadcast_to(allowed, (hq, 1, n)).copy())
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)[:, 0, :].numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_linear_rowwise_equals_matmul():
    x = RNG.standard_normal((5, 33))
    w = RNG.standard_normal((12, 33))
    np.testing.assert_allclose(ops.linear(x, w, rowwise=True), x @ w.T, rtol=1e-12)
    # a row's row-wise result does not depend on the other rows
    a = ops.linear(x, w, rowwise=True)
    b = ops.linear(x[2:3], w, rowwise=True)
    assert np.array_equal(a[2], b[0])
