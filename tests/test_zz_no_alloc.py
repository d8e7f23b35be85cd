"""lora_bgmv_noalloc (no workspace argument: the slice partials live in the
library's static per-device scratch) against lora_bgmv with a workspace, on
two calls in a row, the second with a smaller batch, through the C ABI.

Both forms compute the same sums in the same order (same d_in split, same
shrink and expand bodies), so their outputs are compared bitwise, and each is
also compared with the oracle at the bf16 tolerance.  A batch whose partial
sums exceed the scratch is rejected on the host before any launch.
"""

import numpy as np
import pytest

import oracle
from gpu_helpers import GpuCase, assert_close, require_gpu, say
from lora_workloads import make_config, make_problem

pytestmark = pytest.mark.gpu

LORA_ERR_WORKSPACE = -6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    oracle.build(force=False)
    return require_gpu()


def run_noalloc(c):
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    p = c.prob
    st = B.load().lora_bgmv_noalloc(torch.cuda.current_stream().cuda_stream, B.DTYPES[p.dtype], p.T, c.x.data_ptr(),
                                    c.x.stride(0), p.d_in, c.ids_dev.data_ptr(), c.pool.addr_A_dev.data_ptr(),
                                    c.pool.addr_B_dev.data_ptr(), c.pool.rank_dev.data_ptr(),
                                    c.pool.alpha_dev.data_ptr(), p.n_adapters, c.pool.max_rank, c.y.data_ptr(),
                                    c.y.stride(0), p.d_out)
    torch.cuda.synchronize()
    return st


def run_ws(c):
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    p = c.prob
    ws = B.workspace(B.LORA_OP_BGMV, p.T, p.d_in, p.d_out, c.pool.max_rank)
    B.bgmv(c.x, c.ids_dev, c.pool, c.y, ws, p.dtype)
    torch.cuda.synchronize()


def test_noalloc_matches_workspace_call_twice():
    from segmented_gather_gemm_lora_amd import binding as B

    rng = np.random.default_rng(21)
    ids = rng.integers(-1, 6, 23).astype(np.int32)
    small = make_problem(name="noalloc_small", dtype="bf16", ids=ids, ranks=[8, 16, 32, 4, 64, 12],
                         alphas=[32.0] * 6, d_in=1024, d_out=1536, seed=21, a_std=0.05, b_std=0.05)
    for prob in (make_config(2), small):  # the second call has the smaller batch
        say(f"case noalloc {prob.name} T={prob.T}")
        c_ws, c_na = GpuCase(prob), GpuCase(prob)
        run_ws(c_ws)
        assert run_noalloc(c_na) == 0, B.last_error()
        got, want = B.to_host_bits(c_na.y, "bf16"), B.to_host_bits(c_ws.y, "bf16")
        assert np.array_equal(got, want), f"{prob.name}: noalloc differs from lora_bgmv"
        y_ref, _ = oracle.lora_forward(prob, nthreads=16)
        assert_close(c_na.y_out(), y_ref, "bf16", f"noalloc {prob.name}")


def test_noalloc_rejects_batches_beyond_the_scratch():
    """65536 tokens at rank 256 need 4 slices x 65536 x 256 x 4 B of partial
    sums, more than the scratch: rejected before any launch."""
    from segmented_gather_gemm_lora_amd import binding as B

    FX = 0x7F0000000000
    f = B.load().lora_bgmv_noalloc
    st = f(None, B.LORA_BF16, 65536, FX, 4096, 4096, FX, FX, FX, FX, FX, 8, 256, FX, 4096, 4096)
    assert st == LORA_ERR_WORKSPACE
    assert "scratch" in B.last_error()
