"""Paged adapter storage on the GPU ("Multi-LoRA Serving in Production ..."
(llms.blog), section "Unified Paged Memory"): adapters cut into fixed-size
pages held in scattered frames of one pool, read through per-matrix page
tables.

Paging changes where the adapter bytes live, not what is computed, so:
  * lora_pages_write followed by a host read through the page table gives the
    source bytes back, and frames outside the table are left untouched;
  * lora_sgmv_paged / lora_bgmv_paged return the same bits as lora_sgmv /
    lora_bgmv on the same inputs when both calls pick the same kernel variant
    (same arithmetic, only the load addresses differ);
  * and both match the fp64 oracle at the stated tolerances
    (fp32 |gpu - ref| <= 1e-5 (|ref| + 1); bf16 <= 2e-2 (|ref| + 1e-2)).
Page sizes span 64 B (every row straddles many pages) to 64 KB, frames are
handed out in a seeded random order, and the cases cover the vector and the
scalar load paths (d_in not a multiple of 8, odd ranks).  The paged BGMV's
one-launch form is also run repeatedly on one workspace and with its waits
forced to give up from the host.
"""

import numpy as np
import pytest

import oracle
from gpu_helpers import GpuCase, assert_close, decode, require_gpu, say
from lora_workloads import make_config, make_problem

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    oracle.build(force=False)
    return require_gpu()


@pytest.mark.parametrize("nbytes,page", [(12345, 64), (100000, 16384), (16, 64), (65536 * 3 + 5, 65536)])
def test_pages_write_round_trip(nbytes, page):
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    say(f"case pages_write bytes={nbytes} page={page}")
    rng = np.random.default_rng(nbytes)
    n = B.lora_pages_needed(nbytes, page)
    n_frames = n + 5
    table = rng.permutation(n_frames)[:n].astype(np.int32)
    pages = torch.full((n_frames * page,), 0xA5, dtype=torch.uint8, device="cuda")
    src_host = rng.integers(0, 256, nbytes, dtype=np.uint8)
    src = torch.from_numpy(src_host).cuda()
    tab = torch.from_numpy(np.concatenate([table, np.zeros(4, np.int32)])).cuda()
    st = B.load().lora_pages_write(torch.cuda.current_stream().cuda_stream, pages.data_ptr(), page, tab.data_ptr(),
                                   src.data_ptr(), nbytes)
    assert st == 0, B.last_error()
    torch.cuda.synchronize()
    got = pages.cpu().numpy().reshape(n_frames, page)
    back = np.concatenate([got[f] for f in table])[:nbytes]
    assert np.array_equal(back, src_host)
    # the tail of the last page and frames outside the table are untouched
    last = got[table[-1]][nbytes - (n - 1) * page:]
    assert (last == 0xA5).all()
    for f in sorted(set(range(n_frames)) - set(table.tolist())):
        assert (got[f] == 0xA5).all()


def _paged_vs_dense(prob, page, path, zero_base=True, oracle_check=True, bitwise=True):
    """Runs the dense and the paged call on the same inputs; returns both outputs."""
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    say(f"case paged {prob.name} T={prob.T} d_in={prob.d_in} d_out={prob.d_out} dtype={prob.dtype} "
        f"page={page} path={path}")
    dense = GpuCase(prob, y_init="zero" if zero_base else "stored")
    dense.run(path)
    y_dense = B.to_host_bits(dense.y, prob.dtype)

    pool = B.PagedPool.from_problem(prob, page_bytes=page, shuffle_seed=page + prob.T)
    frames = np.concatenate(pool.frames_A + pool.frames_B)
    assert len(np.unique(frames)) == len(frames)
    y = B.to_device(dense.y_host_in, prob.dtype)
    T, rmax = max(prob.T, 1), max(prob.max_rank, 1)
    if path == "sgmv":
        plan = B.Plan(T).build(prob.ids, pool).upload()
        ws = B.workspace(B.LORA_OP_SGMV, T, prob.d_in, prob.d_out, rmax)
        B.sgmv_paged(dense.x, plan, pool, y, ws, prob.dtype)
    else:
        ws = B.workspace(B.LORA_OP_BGMV, T, prob.d_in, prob.d_out, rmax)
        B.bgmv_paged(dense.x, dense.ids_dev, pool, y, ws, prob.dtype)
    torch.cuda.synchronize()
    y_paged = B.to_host_bits(y, prob.dtype)
    if bitwise:
        assert np.array_equal(y_paged, y_dense), f"{prob.name}: paged and dense outputs differ"
    if oracle_check:
        p = prob
        if zero_base:
            import copy

            p = copy.copy(prob)
            p.y_in = None
        ref, _ = oracle.lora_forward(p, nthreads=16)
        assert_close(decode(y_paged, prob.dtype), ref, prob.dtype, f"{prob.name}/paged/{path}")
    return y_paged, y_dense


def _mixed(dtype, d_in, d_out, ranks, T=300, seed=3):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-1, len(ranks), T).astype(np.int32)
    # a long run of one adapter: a segment of several 16-row blocks
    ids[:130] = 0
    return make_problem(name=f"paged_mixed_{dtype}", dtype=dtype, ids=ids, ranks=ranks,
                        alphas=[2.0 * r for r in ranks], d_in=d_in, d_out=d_out, seed=seed, a_std=0.05, b_std=0.05)


@pytest.mark.parametrize("page", [64, 256, 16384, 65536])
@pytest.mark.parametrize("path", ["sgmv", "bgmv"])
def test_paged_mixed_bf16(page, path):
    _paged_vs_dense(_mixed("bf16", 1024, 1536, [16, 8, 32, 64, 3, 1]), page, path)


@pytest.mark.parametrize("page", [64, 4096])
@pytest.mark.parametrize("path", ["sgmv", "bgmv"])
def test_paged_scalar_paths(page, path):
    """d_in = 1000 (not a multiple of 8: scalar x/A loads), odd ranks (scalar B
    loads), d_out = 300 (ragged column tile); fp32 and bf16."""
    for dtype in ("f32", "bf16"):
        _paged_vs_dense(_mixed(dtype, 1000, 300, [5, 16, 7], T=90, seed=7), page, path)


def test_paged_rank16_long_segments_preset_y():
    """Rank 16, six segments of 100 tokens, y preset to N(0, 1)."""
    rng = np.random.default_rng(11)
    ids = np.repeat(rng.permutation(6), 100).astype(np.int32)
    prob = make_problem(name="paged_chunked", dtype="bf16", ids=ids, ranks=[16] * 6, alphas=[32.0] * 6, d_in=2048,
                        d_out=2048, seed=11)
    _paged_vs_dense(prob, 16384, "sgmv", zero_base=False)


def test_paged_prefill_workload():
    """The prefill workload (4096 tokens, 16 Dirichlet segments, 4096 -> 4096,
    rank 16) from 16 KB pages, against the dense call and the oracle."""
    _paged_vs_dense(make_config(3), 16384, "sgmv")


def test_paged_decode_workload():
    """The decode workload (64 tokens over 32 adapters, rank 16) from 16 KB pages."""
    _paged_vs_dense(make_config(2), 16384, "bgmv")


def test_paged_hetero_workload():
    """The mixed-rank workload (ranks 8..64 unpadded, 4096 -> 14336) from 64 KB
    pages: bitwise equal to the dense call (whose parity with the oracle the
    dense tests establish)."""
    _paged_vs_dense(make_config(4), 65536, "sgmv", zero_base=False, oracle_check=False)


def test_paged_empty_and_no_adapter():
    """A batch where no token has an adapter leaves y untouched."""
    prob = make_problem(name="paged_none", dtype="bf16", ids=[-1] * 40, ranks=[8, 8], alphas=[16.0, 16.0],
                        d_in=256, d_out=256, seed=5)
    yp, yd = _paged_vs_dense(prob, 256, "sgmv", zero_base=False, oracle_check=False)
    assert np.array_equal(yp, prob.y_base())
    yp, yd = _paged_vs_dense(prob, 256, "bgmv", zero_base=False, oracle_check=False)
    assert np.array_equal(yp, prob.y_base())


@pytest.mark.parametrize("path", ["sgmv", "bgmv"])
def test_paged_max_rank(path):
    """Rank 256 (the largest the ABI takes) next to small ranks, 256-byte pages:
    each A row (1 KB) and each B row (512 B) spans several pages, and the
    expand takes the general one-16-rank-step-at-a-time body."""
    rng = np.random.default_rng(31)
    ids = rng.integers(-1, 3, 120).astype(np.int32)
    prob = make_problem(name="paged_rank256", dtype="bf16", ids=ids, ranks=[256, 100, 3], alphas=[64.0, 32.0, 8.0],
                        d_in=512, d_out=520, seed=31, a_std=0.05, b_std=0.05)
    _paged_vs_dense(prob, 256, path)


def test_paged_bgmv_one_launch_give_up_and_repeat():
    """lora_bgmv_paged takes lora_bgmv's one-launch form for the decode
    workload: repeated calls on one workspace (nothing reset) give the dense
    call's bits with the status word at zero; a wait forced to give up from
    the host ends the kernel, sets the status word and leaves y unchanged."""
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    prob = make_config(2)
    dense = GpuCase(prob, y_init="zero")
    dense.run("bgmv")
    y_dense = B.to_host_bits(dense.y, prob.dtype)
    pool = B.PagedPool.from_problem(prob, page_bytes=16384, shuffle_seed=7)
    ws = B.workspace(B.LORA_OP_BGMV, prob.T, prob.d_in, prob.d_out, prob.max_rank)
    y = B.to_device(dense.y_host_in, prob.dtype)
    say("case paged bgmv one-launch repeated calls")
    for _ in range(4):
        y.zero_()
        B.bgmv_paged(dense.x, dense.ids_dev, pool, y, ws, prob.dtype)
        torch.cuda.synchronize()
        assert B.workspace_status(ws) == 0
        assert np.array_equal(B.to_host_bits(y, prob.dtype), y_dense)
    say("case paged bgmv one-launch forced give-up")
    y.zero_()
    B.debug_wait_limit(-1)
    try:
        B.bgmv_paged(dense.x, dense.ids_dev, pool, y, ws, prob.dtype)
        torch.cuda.synchronize()
    finally:
        B.debug_wait_limit(0)
    assert B.workspace_status(ws) == 1
    assert not B.to_host_bits(y, prob.dtype).any(), "a consumer that gave up wrote y"
    B.workspace_clear(ws)
    torch.cuda.synchronize()
    assert B.workspace_status(ws) == 0
