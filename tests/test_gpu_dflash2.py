"""DFlash2 drafter variants on the device through the C ABI, teacher-forced against the oracle
(oracle/dflash2.py): the dynamic convolution through the draft logits of every step (the oracle's drafter
convolves too), and the selector's candidates, transitions and drafts (check_selector in the harness).
Greedy runs must also emit the oracle's greedy stream (the variants change only the drafts)."""
import numpy as np
import pytest
import torch

import synth
from oracle.model import Target
from oracle.spec import Sampling, ar_generate
from synth import weights as sw
from tests.harness import log, run_e2e, tol_of

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,greedy,n_tokens", [("tiny-dflash2", True, 40), ("tiny-dflash2", False, 40),
                                                  ("small-dflash2", True, 24), ("small-dflash2", False, 24)])
def test_dflash2_drafter_e2e(name, greedy, n_tokens):
    cfg = synth.CONFIGS[name]
    if name.startswith("small"):
        from dataclasses import replace
        cfg = replace(cfg, prompt_len=128)
    log(f"[dflash2 e2e] {name} greedy={greedy}")
    W = sw.model_weights(cfg, gain_std=0.1)
    # random factors give transitions far below the logit gaps; scaled up (by a power of two, exact in
    # bf16), the path search decides drafts
    W["d.sel_u"] = W["d.sel_u"] * 32.0
    W["d.sel_v"] = W["d.sel_v"] * 32.0
    sp = synth.GREEDY if greedy else cfg.sampling
    stream, rep, prompt = run_e2e(cfg, W, sp, n_tokens)
    tol = tol_of(cfg)
    le, de = np.array(rep.logits_err), np.array(rep.draft_err)
    log(f"  logits err max {le.max():.3e}, draft logits err max {de.max():.3e}, selector steps {rep.sel_steps}, "
        f"transition err max {max(rep.sel_trans_err):.2e}, tau mean {np.mean(rep.taus):.2f}")
    assert le.max() <= tol and de.max() <= tol
    assert rep.sel_steps == len(rep.taus) > 0
    if greedy and cfg.target.dtype == "fp32":
        t = Target(cfg.target, W, taps=cfg.drafter.taps)
        assert stream == ar_generate(t, prompt.tolist(), n_tokens, Sampling(0.0, 0, 1.0, 1))


def test_dflash2_stochastic_drafts_are_refused():
    from speculative_decoding_dflash_amd import binding as Bd
    from tests.harness import engine, samp
    cfg = synth.CONFIGS["tiny-dflash2"]
    W = sw.model_weights(cfg)
    eng = engine(cfg, W)
    eng.kv_alloc(0, 64)
    P = cfg.prompt_len
    prompt = torch.from_numpy(sw.prompt_ids(cfg.target.vocab, cfg.drafter.mask_id, P, 0)).to("cuda")
    s = samp(cfg.sampling)
    eng.prefill([0], prompt.view(1, -1), [s])
    with pytest.raises(Bd.DflashError) as e:
        eng.draft([0], samplings=[s])
    assert e.value.status == Bd.E_INVAL
