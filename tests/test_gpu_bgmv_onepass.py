"""The one-launch form of lora_bgmv (shrink and expand workgroups in one grid,
handing over through partial sums stored as 64-bit words that carry the tag
of the launch that wrote them).

* parity with the oracle on decode batches whose groups take several 16-token
  passes, and on pools larger than twice the batch (one group per leader
  token);
* equality (bitwise) with the two-kernel form of the same sums (lora_bgmv_paged
  over the same adapters, which always runs as two kernels);
* repeated calls on one workspace, with nothing reset in between, give the
  same result every time and leave the status word at zero;
* a wait forced to give up from the host (lora_debug_wait_limit(-1)) ends the
  kernel normally, sets the status word and leaves y untouched; the next call
  (no reset needed) is correct, and lora_workspace_clear resets the status;
* the call recorded in a graph and replayed several times, with y restored
  eagerly between replays, gives the eager result every time (each replay is
  a launch of its own with its own key).
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


def run_bgmv(c, ws=None):
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    p = c.prob
    if ws is None:
        ws = B.workspace(B.LORA_OP_BGMV, p.T, p.d_in, p.d_out, max(p.max_rank, 1))
    B.bgmv(c.x, c.ids_dev, c.pool, c.y, ws, p.dtype)
    torch.cuda.synchronize()
    return ws


CASES = [
    # name, T, n_adapters (ids uniform), rank, d_in, d_out, seed
    ("multi_pass", 200, 3, 16, 1024, 1024, 1),      # ~67 tokens per adapter: 5 passes
    ("token_groups", 20, 100, 32, 2048, 512, 2),    # pool > 2T: one group per leader token
    ("rank64", 48, 8, 64, 4096, 2048, 3),
    ("rank8_f32", 33, 5, 8, 512, 256, 4),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_onepass_parity(case):
    from segmented_gather_gemm_lora_amd import binding as B

    name, T, n, r, d_in, d_out, seed = case
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, n, T).astype(np.int32)
    ids[rng.random(T) < 0.1] = -1
    dt = "f32" if name.endswith("f32") else "bf16"
    prob = make_problem(name=name, dtype=dt, ids=ids, ranks=[r] * n, alphas=[2.0 * r] * n, d_in=d_in, d_out=d_out,
                        seed=seed, a_std=0.05, b_std=0.05)
    for zero_base in (False, True):
        say(f"case onepass {name} zero_base={zero_base}")
        c = GpuCase(prob, y_init="zero" if zero_base else "stored")
        ws = run_bgmv(c)
        ref_prob = prob
        if zero_base:
            import copy

            ref_prob = copy.copy(prob)
            ref_prob.y_in = None
        y_ref, _ = oracle.lora_forward(ref_prob, nthreads=16)
        y = c.y_out()
        assert_close(y, y_ref, dt, f"onepass {name}")
        none = np.nonzero(prob.ids < 0)[0]
        assert np.array_equal(y[none], decode(c.y_host_in, dt)[none])
        assert B.workspace_status(ws) == 0


def test_onepass_equals_two_kernels():
    """lora_bgmv (one launch) and lora_bgmv_paged (always two kernels, same
    d_in split and bodies) over the same adapters give the same bits."""
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    prob = make_config(2)
    say("case onepass vs two kernels (decode workload)")
    c1 = GpuCase(prob)
    run_bgmv(c1)
    c2 = GpuCase(prob)
    paged = B.PagedPool.from_problem(prob, page_bytes=65536, shuffle_seed=3)
    ws = B.workspace(B.LORA_OP_BGMV, prob.T, prob.d_in, prob.d_out, prob.max_rank)
    B.bgmv_paged(c2.x, c2.ids_dev, paged, c2.y, ws, "bf16")
    torch.cuda.synchronize()
    assert np.array_equal(B.to_host_bits(c1.y, "bf16"), B.to_host_bits(c2.y, "bf16"))


def test_onepass_repeated_calls():
    """Ten calls in a row on one workspace, nothing reset in between: each
    gives the same output and the status word stays zero."""
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    prob = make_config(2)
    c = GpuCase(prob, y_init="zero")
    ws = B.workspace(B.LORA_OP_BGMV, prob.T, prob.d_in, prob.d_out, prob.max_rank)
    say("case onepass repeated calls")
    outs = []
    for _ in range(10):
        c.y.zero_()
        B.bgmv(c.x, c.ids_dev, c.pool, c.y, ws, "bf16")
        torch.cuda.synchronize()
        assert B.workspace_status(ws) == 0
        outs.append(B.to_host_bits(c.y, "bf16"))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_onepass_forced_give_up_ends_normally():
    """The host forces every wait to give up at once: the kernel still ends,
    the status word is set and y is left as it was.  The next call (default
    wait, nothing reset) is correct; lora_workspace_clear resets the status."""
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    prob = make_config(2)
    c = GpuCase(prob)
    y_before = B.to_host_bits(c.y, "bf16")
    ws = B.workspace(B.LORA_OP_BGMV, prob.T, prob.d_in, prob.d_out, prob.max_rank)
    say("case onepass forced give-up")
    B.debug_wait_limit(-1)
    try:
        B.bgmv(c.x, c.ids_dev, c.pool, c.y, ws, "bf16")
        torch.cuda.synchronize()
    finally:
        B.debug_wait_limit(0)
    assert B.workspace_status(ws) == 1
    assert np.array_equal(B.to_host_bits(c.y, "bf16"), y_before), "a consumer that gave up wrote y"
    say("case onepass after a give-up")
    B.bgmv(c.x, c.ids_dev, c.pool, c.y, ws, "bf16")
    torch.cuda.synchronize()
    y_ref, _ = oracle.lora_forward(prob, nthreads=16)
    assert_close(c.y_out(), y_ref, "bf16", "onepass after a give-up")
    assert B.workspace_status(ws) == 1  # sticky until cleared
    B.workspace_clear(ws)
    torch.cuda.synchronize()
    assert B.workspace_status(ws) == 0
    assert bool((ws == 0).all().item())


def test_onepass_graph_replays():
    """lora_bgmv recorded in a graph: three replays, each after y is restored
    by an eager copy, equal the eager call bitwise; the status stays zero."""
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    prob = make_config(2)
    c = GpuCase(prob)
    y0 = c.y.clone()
    ws = B.workspace(B.LORA_OP_BGMV, prob.T, prob.d_in, prob.d_out, prob.max_rank)
    s = torch.cuda.Stream()
    say("case onepass graph: eager")
    with torch.cuda.stream(s):
        B.bgmv(c.x, c.ids_dev, c.pool, c.y, ws, "bf16", stream=s)
    torch.cuda.synchronize()
    eager = B.to_host_bits(c.y, "bf16")
    say("case onepass graph: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        B.bgmv(c.x, c.ids_dev, c.pool, c.y, ws, "bf16", stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"case onepass graph: replay {rep}")
        c.y.copy_(y0)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(B.to_host_bits(c.y, "bf16"), eager), f"replay {rep}"
        assert B.workspace_status(ws) == 0
    del g


@pytest.mark.parametrize("ranks", [[16], [8, 16, 32, 4]], ids=["rank16", "mixed_le32"])
def test_sgmv_onepass_equals_two_kernels(ranks):
    """A small plan runs lora_sgmv in one launch; lora_sgmv_paged over the same
    adapters always runs the two kernels with the same d_in split and sums:
    the outputs are equal bitwise, and both match the oracle."""
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    rng = np.random.default_rng(31)
    n = 12
    ids = rng.integers(-1, n, 96).astype(np.int32)
    rk = [ranks[i % len(ranks)] for i in range(n)]
    prob = make_problem(name="sgmv_small", dtype="bf16", ids=ids, ranks=rk, alphas=[32.0] * n, d_in=2048,
                        d_out=1536, seed=31, a_std=0.05, b_std=0.05)
    say(f"case sgmv one-launch vs two kernels ranks={ranks}")
    c1 = GpuCase(prob)
    timer = B.KernelTimer(8)
    timer.arm(0, 8)
    c1.run("sgmv")
    assert B.KernelTimer.used() == 1, "small plan: one launch"
    timer.disarm()
    timer.close()
    c2 = GpuCase(prob)
    paged = B.PagedPool.from_problem(prob, page_bytes=65536, shuffle_seed=5)
    plan = B.Plan(prob.T).build(prob.ids, paged).upload()
    ws = B.workspace(B.LORA_OP_SGMV, prob.T, prob.d_in, prob.d_out, max(rk))
    B.sgmv_paged(c2.x, plan, paged, c2.y, ws, "bf16")
    torch.cuda.synchronize()
    assert np.array_equal(B.to_host_bits(c1.y, "bf16"), B.to_host_bits(c2.y, "bf16"))
    y_ref, _ = oracle.lora_forward(prob, nthreads=16)
    assert_close(c1.y_out(), y_ref, "bf16", "sgmv one-launch")
