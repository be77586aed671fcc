"""Host-side checks of the C ABI that need no GPU: the library loads, exports every function that
include/dflash.h declares, sizes buffers, and rejects bad configurations before touching the device."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "dflash.h")).read()
    return sorted(set(re.findall(r"^\s*(?:size_t|dflash_status|const char \*)\s*(dflash_\w+)\s*\(", src, re.M)))


def test_header_declares_the_step_calls():
    names = header_functions()
    for n in ("dflash_draft_block", "dflash_verify_block", "dflash_accept_resample", "dflash_kv_alloc",
              "dflash_kv_free"):
        assert n in names


def test_library_exports_every_declared_function():
    from speculative_decoding_dflash_amd import binding as B
    lib = C.CDLL(B.LIB_PATH)
    for n in header_functions():
        assert hasattr(lib, n), n


def _cfgs(**over):
    import synth
    from speculative_decoding_dflash_amd.runner import drafter_cfg, model_cfg
    from speculative_decoding_dflash_amd import binding as B
    c = synth.SMALL
    mc, dc = model_cfg(c.target), drafter_cfg(c.drafter)
    cap = B.Capacity(4, 512, 16, 256, 64)
    for k, v in over.items():
        for o in (mc, dc, cap):
            if hasattr(o, k):
                setattr(o, k, v)
                break
    return mc, dc, cap


def test_sizes_and_validation():
    from speculative_decoding_dflash_amd import binding as B
    mc, dc, cap = _cfgs()
    ws = B.dflash_workspace_bytes(mc, dc, cap)
    assert ws > 0
    # KV pool: layers * pages * 2 * kv_heads * 16 * head_dim * 2 bytes
    assert B.dflash_kv_pool_bytes(mc, 8, cap) == 8 * 256 * 2 * 8 * 16 * 64 * 2
    # the drafter's pool: every page without a window; with one, a ring of
    # ceil((W + 2 B) / 16) + 1 pages per slot, unless that is not smaller
    page = 2 * 8 * 16 * 64 * 2
    dc.window = 0
    assert B.dflash_drafter_pool_bytes(mc, dc, cap) == B.dflash_kv_pool_bytes(mc, dc.layers, cap)
    r200 = -(-(200 + 2 * dc.block_size) // 16) + 1
    for w, pages, ring in ((64, 256, -(-(64 + 2 * dc.block_size) // 16) + 1), (200, 256, r200),
                           (200, 4 * r200, 0), (1000, 256, 0), (4096, 256, 0)):
        dc.window, cap.num_pages = w, pages
        want = dc.layers * cap.max_slots * ring * page if ring else B.dflash_kv_pool_bytes(mc, dc.layers, cap)
        assert B.dflash_drafter_pool_bytes(mc, dc, cap) == want, (w, pages)
    cap.num_pages = 256
    for bad in (dict(head_dim=48), dict(q_heads=12), dict(block_size=0), dict(block_size=17), dict(mask_id=32000),
                dict(page_tokens=8), dict(max_slots=65), dict(window=-1), dict(hidden=1000), dict(dtype=7)):
        mc, dc, cap = _cfgs(**bad)
        assert B.dflash_workspace_bytes(mc, dc, cap) == 0, bad


def test_create_rejects_missing_pointers_without_device_work():
    from speculative_decoding_dflash_amd import binding as B
    mc, dc, cap = _cfgs()
    tw, dw = B.TargetWeights(), B.DrafterWeights()
    out = C.c_void_p()
    st = B.lib.dflash_create(C.byref(mc), C.byref(dc), C.byref(tw), C.byref(dw), C.byref(cap), None, None, None, None,
                             C.byref(out))
    assert st == B.E_INVAL and out.value is None
    assert "missing" in B.dflash_last_error()


def test_null_context_calls_fail_cleanly():
    from speculative_decoding_dflash_amd import binding as B
    assert B.lib.dflash_kv_alloc(None, 0, 16) == B.E_INVAL
    assert B.lib.dflash_kv_free(None, 0) == B.E_INVAL
    assert B.lib.dflash_verify_block(None, None, 1, None, None, 8, 0, 8, None, None) == B.E_INVAL
    assert B.lib.dflash_draft_block(None, None, 1, None, None, None, None) == B.E_INVAL
    assert B.lib.dflash_accept_resample(None, None, 1, None, None, None, 7, None, None, None, None, None) == B.E_INVAL


def test_op_linear_sk_rejects_bad_arguments_on_the_host():
    """dflash_op_linear_sk checks shapes, pointers and the scratch size before any device call (the
    stream and pointers below are never used)."""
    from speculative_decoding_dflash_amd import binding as B
    lib = B.lib
    assert lib.dflash_op_linear_sk_scratch_bytes(0) == 0 and lib.dflash_op_linear_sk_scratch_bytes(48) == 0
    need = lib.dflash_op_linear_sk_scratch_bytes(5120)
    assert need == 1024 * 2 * 512 * 4 + (5120 // 16) * 4
    fake, aligned = 0x10000, 0x100000
    ok = dict(dtype=B.BF16, M=8, N=5120, K=5120, x=fake, w=fake, y=fake, s=aligned, b=need)
    bad = [dict(M=0), dict(M=17), dict(N=48), dict(K=96), dict(K=0), dict(dtype=7), dict(x=None), dict(y=None),
           dict(s=None), dict(s=aligned + 16), dict(b=need - 1), dict(dtype=B.F32, K=96)]
    for over in bad:
        a = {**ok, **over}
        st = lib.dflash_op_linear_sk(None, a["dtype"], a["M"], a["N"], a["K"], a["x"], a["w"], a["y"], a["s"], a["b"])
        assert st == B.E_INVAL, over


@pytest.mark.parametrize("window,block", [(24, 4), (32, 8), (64, 16), (100, 16), (2048, 16)])
def test_drafter_ring_never_loses_a_visible_key(window, block):
    """The drafter's page ring (ring size R read back from dflash_drafter_pool_bytes) against a
    simulation of the positions each draft call touches, over random accept lengths: a prefill, then
    draft / block verify / accept steps.  A draft after an accept of nd drafts of a verify of Q rows at
    n0 injects rows [n0 + max(0, Q - nd - W), n0 + Q), writes its block rows [n, n + B) and reads context
    keys [n - W + 1, n) and the block.  Checked: the positions one call touches are distinct modulo the
    ring's R x 16 positions, and every key a call reads still holds its own position in the ring."""
    from speculative_decoding_dflash_amd import binding as B
    import numpy as np
    mc, dc, cap = _cfgs(window=window, block_size=block)
    cap.max_slots, cap.max_pages_per_seq, cap.num_pages = 2, 4096, 8192
    page = 2 * mc.kv_heads * 16 * mc.head_dim * 2
    nbytes = B.dflash_drafter_pool_bytes(mc, dc, cap)
    R = nbytes // (dc.layers * cap.max_slots * page)
    assert R * dc.layers * cap.max_slots * page == nbytes and R == -(-(window + 2 * block) // 16) + 1
    span = R * 16
    rng = np.random.default_rng(window * 31 + block)
    for trial in range(6):
        ring = {}
        P = int(rng.integers(1, 3 * window + 40))
        n0, Q, nd, n = 0, P, 0, P  # the prefill, accepted: P rows committed
        for step in range(60):
            skip = max(0, Q - nd - window)
            writes = list(range(n0 + skip, n0 + Q)) + list(range(n, n + block))
            reads = list(range(max(0, n - window + 1), n + block))
            touched = set(writes) | set(reads)
            assert len({p % span for p in touched}) == len(touched), (trial, step)
            for p in writes:
                ring[p % span] = p
            for p in reads:
                assert ring.get(p % span) == p, (trial, step, p)
            # block verify at n, accept of tau in 1 .. B (nd = B - 1 drafts)
            n0, Q, nd = n, block, block - 1
            n = n + int(rng.integers(1, block + 1))
