"""Engine: owns the device buffers of one context and sequences the C calls of a decode run.

Only plumbing lives here -- torch allocates the pools, workspace and I/O buffers, and the methods
call the C ABI in the order prefill -> (draft -> verify -> accept)*.  All arithmetic of the step runs
inside libdflash's HIP kernels.
"""
from __future__ import annotations

import ctypes as C
from typing import Dict, List, Optional, Sequence

import torch

from . import binding as B


def model_cfg(t) -> B.ModelCfg:
    return B.ModelCfg(t.layers, t.hidden, t.q_heads, t.kv_heads, t.head_dim, t.ffn, t.vocab, t.rope_theta, t.rms_eps,
                      B.BF16 if t.dtype == "bf16" else B.F32)


def drafter_cfg(d) -> B.DrafterCfg:
    taps = (C.c_int32 * B.MAX_TAPS)(*list(d.taps))
    return B.DrafterCfg(d.layers, len(d.taps), taps, d.block_size, d.mask_id, d.window,
                        getattr(d, "conv_kernel", 0), getattr(d, "conv_group", 16), getattr(d, "selector_top_k", 0),
                        getattr(d, "selector_rank", 256))


def sampling(temperature: float, top_k: int, top_p: float, seed: int) -> B.Sampling:
    return B.Sampling(float(temperature), int(top_k), float(top_p), int(seed))


_LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


class Engine:
    def __init__(self, cfg, weights: Dict[str, torch.Tensor], max_slots: int = 1, max_rows: Optional[int] = None,
                 num_pages: Optional[int] = None, max_pages_per_seq: Optional[int] = None, device: str = "cuda"):
        t, d = cfg.target, cfg.drafter
        self.cfg = cfg
        self.device = torch.device(device)
        self.weights = weights  # keeps the borrowed weights alive
        self.mc = model_cfg(t)
        self.dc = drafter_cfg(d)
        self.B = d.block_size
        max_rows = max_rows or max(cfg.prompt_len, max_slots * d.block_size)
        max_pages_per_seq = max_pages_per_seq or (cfg.prompt_len + cfg.gen_len + 4 * d.block_size) // 16 + 2
        num_pages = num_pages or max_slots * max_pages_per_seq
        self.cap = B.Capacity(max_slots, max_rows, 16, num_pages, max_pages_per_seq)
        ptr = lambda k: weights[k].data_ptr() if k in weights else None  # optional tensors: null when absent
        lw = lambda p: B.LayerWeights(*[weights[p + k].data_ptr() for k in _LAYER_KEYS], ptr(p + "w_conv"))
        self._tl = (B.LayerWeights * t.layers)(*[lw(f"t.L{l}.") for l in range(t.layers)])
        self._dl = (B.LayerWeights * d.layers)(*[lw(f"d.L{j}.") for j in range(d.layers)])
        self.tw = B.TargetWeights(weights["t.embed"].data_ptr(), weights["t.final_norm"].data_ptr(),
                                  weights["t.lm_head"].data_ptr(), self._tl)
        self.dw = B.DrafterWeights(weights["d.fc"].data_ptr(), weights["d.hidden_norm"].data_ptr(),
                                   weights["d.final_norm"].data_ptr(), self._dl, ptr("d.sel_u"), ptr("d.sel_v"))
        u8 = dict(dtype=torch.uint8, device=self.device)
        self.tkv = torch.empty(B.dflash_kv_pool_bytes(self.mc, t.layers, self.cap), **u8)
        self.dkv = torch.empty(B.dflash_drafter_pool_bytes(self.mc, self.dc, self.cap), **u8)
        ws = B.dflash_workspace_bytes(self.mc, self.dc, self.cap)
        if ws == 0:
            raise B.DflashError(B.E_INVAL, "configuration rejected by dflash_workspace_bytes")
        self.ws = torch.empty(ws, **u8)
        self.ctx = B.dflash_create(self.mc, self.dc, self.tw, self.dw, self.cap, self.tkv, self.dkv, self.ws)
        # activation type of the model: fp16 for bf16 models (projection inputs, features, q, KV), fp32 otherwise
        act = torch.float16 if t.dtype == "bf16" else torch.float32
        rows = max(max_rows, 1)
        # target features of the last verify: [rows][taps * hidden] in the activation type
        self.feats = torch.empty(rows * len(d.taps) * t.hidden, dtype=act, device=self.device)
        nl = max_slots * self.B
        self.logits = torch.empty(max(nl, 1) * t.vocab, dtype=torch.float32, device=self.device)
        self.draft_logits = torch.empty(max_slots * max(self.B - 1, 1) * t.vocab, dtype=torch.float32,
                                        device=self.device)
        self.block = torch.zeros(max_slots * self.B, dtype=torch.int32, device=self.device)
        self.out = torch.zeros(max_slots * self.B, dtype=torch.int32, device=self.device)
        self.n_out = torch.zeros(max_slots, dtype=torch.int32, device=self.device)
        self.cand_ids = torch.zeros(nl * B.MAX_TOPK, dtype=torch.int32, device=self.device)
        self.cand_p = torch.zeros(nl * B.MAX_TOPK, dtype=torch.float32, device=self.device)
        # stochastic drafts: the drafter's candidate distributions [max_slots][B-1][MAX_TOPK]
        nq = max_slots * max(self.B - 1, 1) * B.MAX_TOPK
        self.q_ids = torch.zeros(nq, dtype=torch.int32, device=self.device)
        self.q_p = torch.zeros(nq, dtype=torch.float32, device=self.device)
        self._last_verify = None  # (slots, q_len) of the last verify call

    def close(self):
        if self.ctx:
            B.dflash_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------------ calls
    def kv_alloc(self, slot: int, n_tokens: int):
        B.dflash_kv_alloc(self.ctx, slot, n_tokens)

    def kv_free(self, slot: int):
        B.dflash_kv_free(self.ctx, slot)

    def verify(self, slots: Sequence[int], tokens: torch.Tensor, q_len: int, new_sequence: bool, n_logit_rows: int,
               logits: Optional[torch.Tensor] = None):
        B.dflash_verify_block(self.ctx, slots, tokens, q_len, new_sequence, n_logit_rows,
                              self.logits if logits is None else logits, self.feats)
        self._last_verify = (tuple(int(x) for x in slots), int(q_len))

    def accept(self, slots: Sequence[int], n_draft: int, samplings: Sequence[B.Sampling], block=None, cands=False,
               logits: Optional[torch.Tensor] = None, q: bool = False):
        """q: the drafts were drawn from the distributions in q_ids / q_p (stochastic drafts)."""
        lg = self.logits if logits is None else logits
        blk = block if block is not None else (self.block if n_draft > 0 else None)
        ci, cp = (self.cand_ids, self.cand_p) if cands else (None, None)
        if q:
            B.dflash_accept_resample_q(self.ctx, slots, lg, blk, n_draft, samplings, self.q_ids, self.q_p, self.out,
                                       self.n_out, ci, cp)
        else:
            B.dflash_accept_resample(self.ctx, slots, lg, blk, n_draft, samplings, self.out, self.n_out, ci, cp)

    def draft(self, slots: Sequence[int], want_logits: bool = False,
              samplings: Optional[Sequence[B.Sampling]] = None):
        """samplings: draw the drafts from the drafter's filtered distributions (stochastic drafts)."""
        lg = self.draft_logits if want_logits else None
        if samplings is not None:
            B.dflash_draft_block_sampled(self.ctx, slots, self.feats, samplings, self.block, self.q_ids, self.q_p, lg)
        else:
            B.dflash_draft_block(self.ctx, slots, self.feats, self.block, lg)

    def features(self, rows: int) -> torch.Tensor:
        """The target features of the last verify (rows = its batch * q_len) as fp32 [rows, taps, hidden]."""
        nt, H = len(self.cfg.drafter.taps), self.cfg.target.hidden
        return self.feats[:rows * nt * H].float().view(rows, nt, H)

    def status(self):
        B.dflash_device_status(self.ctx)

    # ------------------------------------------------------------------ loops
    def prefill(self, slots: Sequence[int], prompts: torch.Tensor, samplings: Sequence[B.Sampling]):
        """prompts: int32 device tensor [batch, P]."""
        P = prompts.shape[1]
        self.verify(slots, prompts.contiguous(), P, True, 1)
        self.accept(slots, 0, samplings)

    def spec_step(self, slots: Sequence[int], samplings: Sequence[B.Sampling], planted: Optional[torch.Tensor] = None,
                  cands: bool = False, draft_logits: bool = False, stochastic: bool = False):
        """One draft -> verify -> accept step.  planted: optional int32 device [batch, B-1] drafts that
        replace the drafter's (the drafter still runs).  stochastic: drafts drawn from the drafter's
        own distributions and accepted with min(1, p/q)."""
        n = len(slots)
        self.draft(slots, want_logits=draft_logits, samplings=samplings if stochastic else None)
        if planted is not None:
            self.block.view(-1, self.B)[:n, 1:] = planted
        self.verify(slots, self.block, self.B, False, self.B)
        self.accept(slots, self.B - 1, samplings, cands=cands, q=stochastic)

    def capture_spec_step(self, slots: Sequence[int], samplings: Sequence[B.Sampling],
                          planted: Optional[torch.Tensor] = None, stochastic: bool = False) -> "torch.cuda.CUDAGraph":
        """Captures one spec_step (draft -> verify -> accept) into a HIP graph; each replay performs the
        next step.  Every launch parameter of a step is fixed on the host for fixed slots and KV
        allocations (positions, lengths and the accepted tokens live in device memory), so one capture
        serves every later step -- provided the captured launches have the steady-state shapes: the
        step's drafter injection covers as many feature rows as the previous verify wrote, so the last
        verify before the capture must be a block verify over the same slots (an eager spec_step);
        right after a prefill (prompt-length rows, another row stride) or a plain-decoding step (one
        row) the replays would inject the wrong rows, and this raises instead.  Capture records work
        without running it, so the library's host-side bookkeeping advances as if a step had been
        issued; after the capture only replay.  planted: a fixed device tensor copied into the drafts at
        every replay."""
        want = (tuple(int(x) for x in slots), self.B)
        if self._last_verify != want:
            raise RuntimeError(f"capture_spec_step: the last verify was {self._last_verify} (slots, q_len), not a "
                               f"block verify {want} over the same slots; run one eager spec_step first")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.spec_step(slots, samplings, planted=planted, stochastic=stochastic)
        return g

    def ar_step(self, slots: Sequence[int], samplings: Sequence[B.Sampling]):
        """One plain decoding step: verify the anchor alone (the token emitted by the previous prefill or
        ar_step, out[b]) and draw the next token."""
        n = len(slots)
        self.verify(slots, self.out[:n], 1, False, 1)
        self.accept(slots, 0, samplings)
