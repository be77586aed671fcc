"""Workload configurations: model shapes, drafter shapes and run parameters.

Pure data. The five named workloads follow the shapes listed for this
project: a tiny fp32 model for exhaustive checking, a small Qwen3-like
model, a 4B-shaped and a 27B-shaped decoder, and a long-context variant of
the 27B shape.  The drafter of the DFlash write-ups ("Qwen3.8-27B-DFlash2",
page 3, section "结构一览") is five Qwen3-structured layers of the target's
width, a 2048-token sliding window, and taps at target layers
5/19/33/47/61; its embedding table and LM head are the target's own.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import List, Optional, Tuple


@dataclass(frozen=True)
class DecoderCfg:
    layers: int
    hidden: int
    q_heads: int
    kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rope_theta: float
    rms_eps: float = 1e-6
    dtype: str = "bf16"  # "bf16" or "fp32": storage type of weights and activations

    @property
    def q_dim(self) -> int:
        return self.q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.kv_heads * self.head_dim

    def layer_params(self) -> int:
        h = self.hidden
        return h * (self.q_dim + 2 * self.kv_dim) + self.q_dim * h + 3 * h * self.ffn


@dataclass(frozen=True)
class DrafterCfg:
    layers: int
    taps: Tuple[int, ...]  # 0-indexed target layers whose output residual stream is injected
    block_size: int
    mask_id: int
    window: int = 0  # sliding window in tokens; 0 means unbounded
    # DFlash2 variants (oracle/dflash2.py): dynamic convolution taps along the block (0: off) and the
    # channels sharing a tap set; selector candidates per draft position (0: argmax drafts) and the rank
    # of its transition factors
    conv_kernel: int = 0
    conv_group: int = 16
    selector_top_k: int = 0
    selector_rank: int = 256


@dataclass(frozen=True)
class SamplingCfg:
    temperature: float = 1.0  # 0 means greedy
    top_k: int = 20
    top_p: float = 0.95
    seed: int = 1


@dataclass(frozen=True)
class RunCfg:
    name: str
    target: DecoderCfg
    drafter: DrafterCfg
    prompt_len: int
    gen_len: int
    concurrency: int = 1
    sampling: SamplingCfg = field(default_factory=SamplingCfg)
    weight_seed: int = 0
    weight_std: float = 0.02
    # long-context workload: per-request prompt length drawn uniformly from this range (inclusive)
    prompt_len_range: Optional[Tuple[int, int]] = None
    page_tokens: int = 16
    corruption_rates: Tuple[float, ...] = ()


GREEDY = SamplingCfg(temperature=0.0, top_k=0, top_p=1.0, seed=1)

TINY = RunCfg(
    name="tiny",
    target=DecoderCfg(layers=2, hidden=128, q_heads=4, kv_heads=4, head_dim=32, ffn=256, vocab=512,
                      rope_theta=1e4, dtype="fp32"),
    drafter=DrafterCfg(layers=1, taps=(1,), block_size=4, mask_id=511, window=0),
    prompt_len=32, gen_len=64,
    sampling=SamplingCfg(temperature=1.0, top_k=20, top_p=0.95, seed=1),
)

SMALL = RunCfg(
    name="small",
    target=DecoderCfg(layers=8, hidden=1024, q_heads=16, kv_heads=8, head_dim=64, ffn=2816, vocab=32000,
                      rope_theta=1e6),
    drafter=DrafterCfg(layers=2, taps=(1, 4, 7), block_size=8, mask_id=31999, window=0),
    prompt_len=512, gen_len=512,
    corruption_rates=(0.0, 0.1, 0.3, 0.6),
)

B4 = RunCfg(
    name="4b",
    target=DecoderCfg(layers=36, hidden=2560, q_heads=32, kv_heads=8, head_dim=128, ffn=9728, vocab=151936,
                      rope_theta=1e6),
    drafter=DrafterCfg(layers=5, taps=(5, 12, 19, 26, 33), block_size=8, mask_id=151935, window=0),
    prompt_len=2048, gen_len=1024,
)

B27 = RunCfg(
    name="27b",
    target=DecoderCfg(layers=64, hidden=5120, q_heads=40, kv_heads=8, head_dim=128, ffn=17408, vocab=151936,
                      rope_theta=1e6),
    drafter=DrafterCfg(layers=5, taps=(5, 19, 33, 47, 61), block_size=8, mask_id=151935, window=2048),
    prompt_len=1024, gen_len=1024,
)

LONG = replace(B27, name="27b-long", concurrency=32, prompt_len=8192, prompt_len_range=(4096, 8192),
               gen_len=512)

# The same workloads with the DFlash2 drafter variants switched on (2-tap dynamic convolution over groups
# of 16 channels, 16 selector candidates; rank 256, or 32 at the tiny width).
def dflash2(cfg: RunCfg, rank: int = 256) -> RunCfg:
    return replace(cfg, name=cfg.name + "-dflash2",
                   drafter=replace(cfg.drafter, conv_kernel=2, conv_group=16, selector_top_k=16, selector_rank=rank))


TINY2 = dflash2(TINY, rank=32)
SMALL2 = dflash2(SMALL)
B27_2 = dflash2(B27)

CONFIGS = {c.name: c for c in (TINY, SMALL, B4, B27, LONG, TINY2, SMALL2, B27_2)}


def with_layers(cfg: RunCfg, target_layers: int, drafter_layers: int, taps: Tuple[int, ...]) -> RunCfg:
    """Same widths, fewer layers: used by parity tests at full width."""
    return replace(cfg, target=replace(cfg.target, layers=target_layers),
                   drafter=replace(cfg.drafter, layers=drafter_layers, taps=taps))


def tensor_shapes(t: DecoderCfg, d: DrafterCfg) -> List[Tuple[str, Tuple[int, ...], str]]:
    """Logical tensors of a target/drafter pair: (name, shape, kind).

    kind is "w" for a projection or table drawn from N(0, std) and "g" for an
    RMSNorm gain.  Projections are stored [out, in] row-major.  The drafter
    has no embedding table or LM head of its own: it reuses the target's.
    """
    out: List[Tuple[str, Tuple[int, ...], str]] = []
    h, f = t.hidden, t.ffn

    def layer(prefix: str):
        out.extend([
            (prefix + "attn_norm", (h,), "g"),
            (prefix + "wq", (t.q_dim, h), "w"),
            (prefix + "wk", (t.kv_dim, h), "w"),
            (prefix + "wv", (t.kv_dim, h), "w"),
            (prefix + "q_norm", (t.head_dim,), "g"),
            (prefix + "k_norm", (t.head_dim,), "g"),
            (prefix + "wo", (h, t.q_dim), "w"),
            (prefix + "ffn_norm", (h,), "g"),
            (prefix + "w_gate", (f, h), "w"),
            (prefix + "w_up", (f, h), "w"),
            (prefix + "w_down", (h, f), "w"),
        ])

    out.append(("t.embed", (t.vocab, h), "w"))
    for l in range(t.layers):
        layer(f"t.L{l}.")
    out.append(("t.final_norm", (h,), "g"))
    out.append(("t.lm_head", (t.vocab, h), "w"))
    out.append(("d.fc", (h, len(d.taps) * h), "w"))
    out.append(("d.hidden_norm", (h,), "g"))
    for j in range(d.layers):
        layer(f"d.L{j}.")
        if d.conv_kernel:
            out.append((f"d.L{j}.w_conv", (d.conv_kernel * h // d.conv_group, h), "w"))
    out.append(("d.final_norm", (h,), "g"))
    if d.selector_top_k:
        out.append(("d.sel_u", (d.selector_rank, h), "w"))
        out.append(("d.sel_v", (d.selector_rank, h), "w"))
    return out
