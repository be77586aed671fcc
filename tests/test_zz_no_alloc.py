"""dflash_op_linear_sk_noalloc (the stream-K projection with the library's static scratch, for callers
that cannot allocate) against dflash_op_linear_sk (caller scratch): bit for bit on two calls in a row,
the second smaller, and within float64-matmul tolerance; sizes beyond the static limit are refused."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _inputs(M, N, K, dtype, seed):
    rng = np.random.default_rng(seed)
    xt, wt = (torch.float16, torch.bfloat16) if dtype == "bf16" else (torch.float32, torch.float32)
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(xt).cuda()
    w = torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).to(wt).cuda()
    return x, w


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_equals_workspace_entry_point(dtype):
    from speculative_decoding_dflash_amd import binding as Bd
    dt = Bd.BF16 if dtype == "bf16" else Bd.F32
    for M, N, K in [(8, 5120, 17408), (3, 640, 256)]:  # the second call smaller than the first
        print(f"[noalloc] {dtype} {M}x{N}x{K}", flush=True)
        x, w = _inputs(M, N, K, dtype, M + N + K)
        scratch = torch.empty(Bd.dflash_op_linear_sk_scratch_bytes(N), dtype=torch.uint8, device="cuda")
        y_ws = torch.zeros(M * N, dtype=torch.float32, device="cuda")
        y_st = torch.full((M * N,), float("nan"), dtype=torch.float32, device="cuda")
        Bd.dflash_op_linear_sk(dt, M, N, K, x, w, y_ws, scratch)
        Bd.dflash_op_linear_sk_noalloc(dt, M, N, K, x, w, y_st)
        torch.cuda.synchronize()
        assert torch.equal(y_ws, y_st)
        ref = x.double().cpu().numpy() @ w.double().cpu().numpy().T
        err = np.abs(y_st.view(M, N).cpu().numpy() - ref).max() / np.abs(ref).max()
        assert err < 1e-5


def test_noalloc_refuses_beyond_limits():
    from speculative_decoding_dflash_amd import binding as Bd
    x, w = _inputs(4, 256, 256, "bf16", 0)
    y = torch.zeros(4 * 256, dtype=torch.float32, device="cuda")
    for M, N in [(17, 256), (4, 131072 + 32), (4, 48)]:
        with pytest.raises(Bd.DflashError) as e:
            Bd.dflash_op_linear_sk_noalloc(Bd.BF16, M, N, 256, x, w, y)
        assert e.value.status == Bd.E_INVAL
