"""Pins of the oracle's composed forwards against an independent torch (CPU, float64) formulation:
SDPA with library causal / explicit masks, torch's rms_norm, and RoPE written as a complex rotation."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle.model import Drafter, Target
from synth import weights as sw


def _t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def rope_complex(x, pos, theta):
    """x: [n, h, d] rotated as complex numbers (x_i + j x_{i+d/2}) * exp(j pos theta^(-2i/d))."""
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-2.0 * torch.arange(half, dtype=torch.float64) / d)
    ang = pos[:, None].double() * inv[None, :]
    z = torch.complex(x[..., :half], x[..., half:]) * torch.polar(torch.ones_like(ang), ang)[:, None, :]
    return torch.cat([z.real, z.imag], dim=-1)


def torch_layer(W, p, cfg, x, pos, attn_fn):
    eps = cfg.rms_eps
    hq, hkv, d = cfg.q_heads, cfg.kv_heads, cfg.head_dim
    xn = F.rms_norm(x, (cfg.hidden,), weight=_t(W[p + "attn_norm"]), eps=eps)
    q = F.linear(xn, _t(W[p + "wq"])).view(-1, hq, d)
    k = F.linear(xn, _t(W[p + "wk"])).view(-1, hkv, d)
    v = F.linear(xn, _t(W[p + "wv"])).view(-1, hkv, d)
    q = rope_complex(F.rms_norm(q, (d,), weight=_t(W[p + "q_norm"]), eps=eps), pos, cfg.rope_theta)
    k = rope_complex(F.rms_norm(k, (d,), weight=_t(W[p + "k_norm"]), eps=eps), pos, cfg.rope_theta)
    a = attn_fn(q, k, v)  # [n, hq, d]
    x = x + F.linear(a.reshape(len(x), -1), _t(W[p + "wo"]))
    xn = F.rms_norm(x, (cfg.hidden,), weight=_t(W[p + "ffn_norm"]), eps=eps)
    h = F.silu(F.linear(xn, _t(W[p + "w_gate"]))) * F.linear(xn, _t(W[p + "w_up"]))
    return x + F.linear(h, _t(W[p + "w_down"])), k, v


def sdpa(q, k, v, mask=None, causal=False):
    # [n, h, d] -> [h, n, d]; grouped heads via enable_gqa
    out = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1),
                                         attn_mask=mask, is_causal=causal, enable_gqa=True)
    return out.transpose(0, 1)


def small_cfg():
    t = synth.DecoderCfg(layers=3, hidden=64, q_heads=4, kv_heads=2, head_dim=16, ffn=96, vocab=97,
                         rope_theta=1e4, dtype="fp32")
    d = synth.DrafterCfg(layers=2, taps=(0, 2), block_size=5, mask_id=96, window=7)
    return synth.RunCfg(name="m", target=t, drafter=d, prompt_len=20, gen_len=8, weight_std=0.2)


def test_target_forward_matches_torch_causal():
    cfg = small_cfg()
    W = sw.model_weights(cfg, gain_std=0.2)
    tg = Target(cfg.target, W, taps=cfg.drafter.taps)
    toks = sw.prompt_ids(97, 96, 20, 0)
    logits, feats = tg.forward(tg.new_cache(), toks, 0)
    x = _t(W["t.embed"][toks])
    pos = torch.arange(20)
    ref_feats = []
    for l in range(cfg.target.layers):
        x, _, _ = torch_layer(W, f"t.L{l}.", cfg.target, x, pos, lambda q, k, v: sdpa(q, k, v, causal=True))
        if l in cfg.drafter.taps:
            ref_feats.append(x)
    ref = F.linear(F.rms_norm(x, (64,), weight=_t(W["t.final_norm"]), eps=1e-6), _t(W["t.lm_head"]))
    np.testing.assert_allclose(logits, ref.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(feats, torch.stack(ref_feats, 1).numpy(), rtol=1e-9, atol=1e-11)
    # incremental: the prompt split into a prefix and two blocks gives the same last rows
    c = tg.new_cache()
    tg.forward(c, toks[:11], 0)
    tg.forward(c, toks[11:15], 11)
    z, _ = tg.forward(c, toks[15:], 15)
    np.testing.assert_allclose(z, logits[15:], rtol=1e-9, atol=1e-11)


@pytest.mark.parametrize("window", [0, 7, 30])
def test_drafter_matches_torch_masks(window):
    """Injected context K/V (fc -> RMSNorm -> per-layer k/v, k-norm, RoPE) plus a bidirectional block,
    with the per-query sliding window, against SDPA with an explicit mask."""
    from dataclasses import replace
    cfg = small_cfg()
    cfg = replace(cfg, drafter=replace(cfg.drafter, window=window))
    W = sw.model_weights(cfg, gain_std=0.2)
    tg = Target(cfg.target, W, taps=cfg.drafter.taps)
    dr = Drafter(cfg.target, cfg.drafter, W)
    toks = sw.prompt_ids(97, 96, 20, 0)
    _, feats = tg.forward(tg.new_cache(), toks, 0)
    cache = dr.new_cache()
    dr.inject(cache, feats, 0)
    n, B, anchor = 20, 5, 42
    got = dr.draft_logits(cache, anchor, n)

    tc, dc = cfg.target, cfg.drafter
    c = F.rms_norm(F.linear(_t(feats.reshape(n, -1)), _t(W["d.fc"])), (64,), weight=_t(W["d.hidden_norm"]), eps=1e-6)
    x = _t(W["t.embed"][[anchor] + [96] * (B - 1)])
    qpos = torch.arange(n, n + B)
    keys = torch.arange(n + B)
    allowed = (keys[None, :] >= n) | ((window <= 0) | (qpos[:, None] - keys[None, :] < window))
    for j in range(dc.layers):
        p = f"d.L{j}."
        kc = F.linear(c, _t(W[p + "wk"])).view(n, tc.kv_heads, tc.head_dim)
        vc = F.linear(c, _t(W[p + "wv"])).view(n, tc.kv_heads, tc.head_dim)
        kc = rope_complex(F.rms_norm(kc, (tc.head_dim,), weight=_t(W[p + "k_norm"]), eps=1e-6), torch.arange(n),
                          tc.rope_theta)

        def attn(q, k, v, kc=kc, vc=vc):
            return sdpa(q, torch.cat([kc, k]), torch.cat([vc, v]), mask=allowed[None].expand(tc.q_heads, B, n + B))

        x, _, _ = torch_layer(W, p, tc, x, qpos, attn)
    ref = F.linear(F.rms_norm(x[1:], (64,), weight=_t(W["d.final_norm"]), eps=1e-6), _t(W["t.lm_head"]))
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-9, atol=1e-11)
