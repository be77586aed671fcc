"""Error paths and state rules of the C boundary on the device: page-pool exhaustion leaves other slots
untouched, out-of-order calls are refused before anything is enqueued, a token id outside the
vocabulary is caught by the device-side bounds check and reported by dflash_device_status, freed
pages are reused, and repeated runs are bit-identical."""
import numpy as np
import pytest
import torch

import synth
from harness import engine, log, samp
from synth import weights as sw

pytestmark = pytest.mark.gpu


def _greedy_run(eng, slot, prompt, n, g):
    """Greedy speculative decoding of one slot: (tokens, verify logits of every step)."""
    B, V = eng.B, eng.cfg.target.vocab
    eng.prefill([slot], prompt.view(1, -1), [g])
    toks, rows = [int(eng.out[0])], []
    while len(toks) < n:
        eng.spec_step([slot], [g])
        tau = int(eng.n_out[0])
        toks.extend(int(x) for x in eng.out[:tau].cpu().numpy())
        rows.append(eng.logits[:B * V].cpu().clone())
    eng.status()
    return toks[:n], rows


def _prompt(cfg, request, P=None):
    P = P or cfg.prompt_len
    return torch.from_numpy(sw.prompt_ids(cfg.target.vocab, cfg.drafter.mask_id, P, request)).to("cuda")


def test_nomem_leaves_other_slots_intact():
    """A reservation the pool cannot hold fails with DFLASH_E_NOMEM and changes nothing: the slot that
    asked holds no pages (its calls are refused with DFLASH_E_STATE), and the slot already decoding
    emits exactly the stream it emits alone."""
    from speculative_decoding_dflash_amd import binding as Bd
    cfg = synth.TINY
    W = sw.model_weights(cfg)
    P, B, n = cfg.prompt_len, cfg.drafter.block_size, 32
    need = (P + n + 4 * B + 15) // 16
    g = samp(synth.GREEDY)
    prompt = _prompt(cfg, 0)
    eng = engine(cfg, W, max_slots=2, num_pages=need + 2, max_pages_per_seq=need + 2)
    eng.kv_alloc(0, P + n + 4 * B)
    ref, _ = _greedy_run(eng, 0, prompt, n, g)
    eng.close()

    eng = engine(cfg, W, max_slots=2, num_pages=need + 2, max_pages_per_seq=need + 2)
    eng.kv_alloc(0, P + n + 4 * B)
    with pytest.raises(Bd.DflashError) as e:
        eng.kv_alloc(1, 16 * (need + 1))
    assert e.value.status == Bd.E_NOMEM
    log(f"  E_NOMEM: {e.value}")
    with pytest.raises(Bd.DflashError) as e:
        eng.verify([1], _prompt(cfg, 1), P, True, 1)
    assert e.value.status == Bd.E_STATE
    eng.kv_alloc(1, 2 * 16)  # what is left still serves another slot
    got, _ = _greedy_run(eng, 0, prompt, n, g)
    assert got == ref
    eng.close()


def test_out_of_order_calls_refused():
    """Calls out of order for their slots return DFLASH_E_STATE and enqueue nothing: an accept with no
    verify before it, a draft on slots other than the last verify's, a decoding verify of a slot that
    was never prefilled; the context then decodes normally."""
    from speculative_decoding_dflash_amd import binding as Bd
    cfg = synth.TINY
    W = sw.model_weights(cfg)
    P, B, n = cfg.prompt_len, cfg.drafter.block_size, 24
    g = samp(synth.GREEDY)
    ref_eng = engine(cfg, W, max_slots=2)
    ref_eng.kv_alloc(0, P + n + 4 * B)
    ref, _ = _greedy_run(ref_eng, 0, _prompt(cfg, 0), n, g)
    ref_eng.close()

    eng = engine(cfg, W, max_slots=2)
    for s_ in (0, 1):
        eng.kv_alloc(s_, P + n + 4 * B)
    with pytest.raises(Bd.DflashError) as e:  # decoding verify of a slot never prefilled
        eng.verify([0], eng.block, B, False, B)
    assert e.value.status == Bd.E_STATE
    eng.verify([1], _prompt(cfg, 1), P, True, 1)
    eng.accept([1], 0, [g])
    with pytest.raises(Bd.DflashError) as e:  # a second accept of the same verify
        eng.accept([1], 0, [g])
    assert e.value.status == Bd.E_STATE
    with pytest.raises(Bd.DflashError) as e:  # draft for slot 0 after a verify of slot 1
        Bd.dflash_draft_block(eng.ctx, [0], eng.feats, eng.block, None)
    assert e.value.status == Bd.E_STATE
    eng.status()
    got, _ = _greedy_run(eng, 0, _prompt(cfg, 0), n, g)
    assert got == ref
    eng.close()


def test_windowed_drafter_page_ring():
    """A windowed drafter recycles a ring of ceil((W + 2 B) / 16) + 1 pages per slot: its pool is that
    size (the full pool when the page pool is no larger than the rings), a draft straight after a
    verify -- no accept to say which rows were committed -- is refused with DFLASH_E_STATE, and a
    greedy run whose context wraps the ring several times is bit-identical (tokens and every verify
    logit) to the same run on a context whose drafter uses the target's page ids."""
    from dataclasses import replace

    from speculative_decoding_dflash_amd import binding as Bd
    cfg = replace(synth.TINY, drafter=replace(synth.TINY.drafter, window=24), prompt_len=96)
    W = sw.model_weights(cfg)
    P, B, n = cfg.prompt_len, cfg.drafter.block_size, 40
    R = -(-(24 + 2 * B) // 16) + 1
    g = samp(synth.GREEDY)
    runs = []
    for ring in (True, False):
        eng = engine(cfg, W, max_slots=4, **({} if ring else dict(num_pages=4 * R)))
        page = 2 * cfg.target.kv_heads * 16 * cfg.target.head_dim * 4
        full = Bd.dflash_kv_pool_bytes(eng.mc, cfg.drafter.layers, eng.cap)
        assert eng.dkv.numel() == (cfg.drafter.layers * 4 * R * page if ring else full)
        eng.kv_alloc(0, P + n + 2 * B)
        if ring:  # (the pool without the ring holds one such slot)
            eng.kv_alloc(1, P + 2 * B)
            eng.verify([1], _prompt(cfg, 1), P, True, 1)
            with pytest.raises(Bd.DflashError) as e:
                Bd.dflash_draft_block(eng.ctx, [1], eng.feats, eng.block, None)
            assert e.value.status == Bd.E_STATE
            eng.accept([1], 0, [g])
            Bd.dflash_draft_block(eng.ctx, [1], eng.feats, eng.block, None)
        runs.append(_greedy_run(eng, 0, _prompt(cfg, 0), n, g))
        eng.close()
    assert P + n > 2 * R * 16 and runs[0][0] == runs[1][0]
    assert all(torch.equal(a, b) for a, b in zip(runs[0][1], runs[1][1]))
    log(f"[drafter ring] {R} pages per slot, {len(runs[0][1])} verify steps bit-identical")


def test_bad_token_raises_device_flag():
    """A token id outside [0, vocab) is a condition only the device sees: the verify is accepted on the
    host, the row preparation substitutes a safe id and raises its sticky flag, dflash_device_status
    returns DFLASH_E_DEVICE naming it and clears it; the next status is clean."""
    from speculative_decoding_dflash_amd import binding as Bd
    cfg = synth.TINY
    W = sw.model_weights(cfg)
    P, V = cfg.prompt_len, cfg.target.vocab
    eng = engine(cfg, W)
    eng.kv_alloc(0, P + 16)
    toks = _prompt(cfg, 0).clone()
    toks[5] = V
    eng.verify([0], toks, P, True, 1)
    with pytest.raises(Bd.DflashError) as e:
        eng.status()
    assert e.value.status == Bd.E_DEVICE and "token id out of range" in str(e.value)
    log(f"  {e.value}")
    eng.status()
    eng.close()


def test_free_then_realloc_reuses_pages():
    """With a pool of exactly one sequence's pages, a slot's pages go back to the pool on
    dflash_kv_free and another slot's reservation takes them; that slot, prefilled with the same
    prompt, emits the same stream and the same verify logits bit for bit (the reused pages hold the
    first slot's stale K/V, which no read reaches)."""
    cfg = synth.TINY
    W = sw.model_weights(cfg)
    P, B, n = cfg.prompt_len, cfg.drafter.block_size, 32
    need = (P + n + 4 * B + 15) // 16
    g = samp(synth.GREEDY)
    prompt = _prompt(cfg, 0)
    eng = engine(cfg, W, max_slots=2, num_pages=need, max_pages_per_seq=need)
    eng.kv_alloc(0, 16 * need)
    a_toks, a_rows = _greedy_run(eng, 0, prompt, n, g)
    eng.kv_free(0)
    eng.kv_alloc(1, 16 * need)
    b_toks, b_rows = _greedy_run(eng, 1, prompt, n, g)
    assert a_toks == b_toks
    assert len(a_rows) == len(b_rows) and all(torch.equal(x, y) for x, y in zip(a_rows, b_rows))
    eng.close()


def test_repeat_runs_bit_identical():
    """Two contexts given the same inputs produce the same sampled stream, drafts and logits bit for bit
    (small model, bf16, T = 1 / top-k 20 / top-p 0.95): every reduction runs in a fixed order."""
    from harness import small_short
    cfg = small_short()
    W = sw.model_weights(cfg)
    P, B, V = cfg.prompt_len, cfg.drafter.block_size, cfg.target.vocab
    s = samp(cfg.sampling)

    def run():
        eng = engine(cfg, W)
        eng.kv_alloc(0, P + 20 * B)
        eng.prefill([0], _prompt(cfg, 0).view(1, -1), [s])
        rec = []
        for _ in range(12):
            eng.spec_step([0], [s])
            tau = int(eng.n_out[0])
            rec.append((eng.out[:tau].cpu().clone(), eng.block[:B].cpu().clone(), eng.logits[:B * V].cpu().clone()))
        eng.status()
        eng.close()
        return rec

    a, b = run(), run()
    for i, (x, y) in enumerate(zip(a, b)):
        assert all(torch.equal(u, v) for u, v in zip(x, y)), f"step {i} differs"
