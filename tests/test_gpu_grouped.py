"""Parity of the grouped BGMV entry (several projections of a layer in one
launch, or one shrink launch and one expand launch when a projection does not
fit the one-launch form) with the fp64 oracle, through the C ABI.

Every projection is its own problem (x, y, d_in, d_out, adapter tables) with
the same per-token adapter ids; each is checked against the oracle of that
problem at the usual tolerances (fp32 |gpu - ref| <= 1e-5 (|ref| + 1); bf16
|gpu - ref| <= 2e-2 (|ref| + 1e-2)), rows of tokens without an adapter must be
untouched, and where every projection takes the same kernel variant as a
single lora_bgmv call the bits must equal that call's.  The one-launch form is
also run repeatedly on one workspace and with its waits forced to give up from
the host (the kernel must still end, set the status word and leave y as it
was).
"""

import numpy as np
import pytest

import oracle
from gpu_helpers import GpuCase, assert_close, decode, require_gpu, say
from lora_workloads import f32_to_bf16_bits, make_integer_problem, make_problem

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    oracle.build(force=False)
    return require_gpu()


def projections(ids, specs, dtype, seed, share_x=False):
    """One problem per projection spec (d_in, d_out, ranks), all with `ids`;
    with share_x every projection reads the first one's x."""
    probs = []
    for p, (d_in, d_out, ranks) in enumerate(specs):
        prob = make_problem(name=f"proj{p}", dtype=dtype, ids=ids, ranks=ranks, alphas=[2.0 * r for r in ranks],
                            d_in=d_in, d_out=d_out, seed=seed + 17 * p, a_std=0.05, b_std=0.05)
        if share_x and p > 0:
            assert d_in == probs[0].d_in
            prob.x = probs[0].x
        probs.append(prob)
    return probs


def run_grouped(probs, share_x=False):
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    cases = [GpuCase(p) for p in probs]
    if share_x:
        for c in cases[1:]:
            c.x = cases[0].x
    xs, pools, ys = [c.x for c in cases], [c.pool for c in cases], [c.y for c in cases]
    projs = B.proj_array(xs, pools, ys)
    ws = B.bgmv_grouped_workspace(probs[0].T, projs)
    B.bgmv_grouped(xs, cases[0].ids_dev, pools, ys, ws, probs[0].dtype, projs=projs)
    torch.cuda.synchronize()
    return cases


def check_against_oracle(probs, cases, what):
    for p, (prob, c) in enumerate(zip(probs, cases)):
        y = c.y_out()
        y_ref, _ = oracle.lora_forward(prob, nthreads=16)
        assert_close(y, y_ref, prob.dtype, f"{what}/proj{p}")
        none = np.nonzero(prob.ids < 0)[0]
        if len(none):
            assert np.array_equal(y[none], decode(c.y_host_in, prob.dtype)[none]), f"{what}/proj{p}: unadapted rows"


def single_bits(prob):
    """The same projection through one lora_bgmv call."""
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    c = GpuCase(prob)
    ws = B.workspace(B.LORA_OP_BGMV, prob.T, prob.d_in, prob.d_out, max(prob.max_rank, 1))
    B.bgmv(c.x, c.ids_dev, c.pool, c.y, ws, prob.dtype)
    torch.cuda.synchronize()
    return B.to_host_bits(c.y, prob.dtype)


def test_qkv_shared_x():
    """q, k, v of a decode batch (64 tokens, 32 adapters of rank 16, d_in 4096,
    d_out 4096 / 1024 / 1024): one shrink and one expand launch."""
    from segmented_gather_gemm_lora_amd import binding as B

    rng = np.random.default_rng(5)
    ids = rng.integers(0, 32, 64).astype(np.int32)
    specs = [(4096, 4096, [16] * 32), (4096, 1024, [16] * 32), (4096, 1024, [16] * 32)]
    probs = projections(ids, specs, "bf16", seed=50, share_x=True)
    say("case grouped qkv shared x")
    cases = run_grouped(probs, share_x=True)
    check_against_oracle(probs, cases, "qkv")
    say("case grouped qkv vs single calls")
    for p, (prob, c) in enumerate(zip(probs, cases)):
        assert np.array_equal(B.to_host_bits(c.y, "bf16"), single_bits(prob)), f"proj{p} differs from lora_bgmv"


MIXED = [
    # name, dtype, T, n_adapters, none_frac, specs (d_in, d_out, ranks per adapter seed), seed
    ("slot_bf16", "bf16", 37, 20, 0.15, [(512, 1000), (1024, 336), (200, 130)], 61),
    ("slot_f32", "f32", 29, 12, 0.1, [(256, 400), (136, 264), (512, 72)], 62),
    ("token_major_bf16", "bf16", 24, 100, 0.1, [(1024, 512), (1024, 2048)], 63),
    ("eight_projections", "bf16", 16, 9, 0.0, [(128 * (1 + p % 3), 96 + 32 * p) for p in range(8)], 64),
]


@pytest.mark.parametrize("case", MIXED, ids=[m[0] for m in MIXED])
def test_mixed_projections(case):
    """Different d_in, d_out (some not multiples of 16), heterogeneous ranks
    per projection; slot-major and per-token grids; fp32 and bf16."""
    name, dtype, T, n_adapters, none_frac, dims, seed = case
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, n_adapters, T).astype(np.int32)
    ids[rng.random(T) < none_frac] = -1
    specs = [(d_in, d_out, list(rng.choice([1, 4, 8, 13, 16, 32, 64], n_adapters))) for d_in, d_out in dims]
    probs = projections(ids, specs, dtype, seed=seed)
    say(f"case grouped {name}")
    cases = run_grouped(probs)
    check_against_oracle(probs, cases, name)


def test_integer_bitwise():
    """Entries in {-1,0,1}, scale 1, three projections: every sum is exact, so
    each bf16 output equals the exact result rounded once."""
    from segmented_gather_gemm_lora_amd import binding as B

    probs = [make_integer_problem(seed=71, dtype="bf16", T=40, d_in=d_in, d_out=d_out, n_adapters=5, none_frac=0.1)
             for d_in, d_out in [(200, 333), (64, 48), (512, 96)]]
    assert all(np.array_equal(p.ids, probs[0].ids) for p in probs)
    say("case grouped integer")
    cases = run_grouped(probs)
    for p, (prob, c) in enumerate(zip(probs, cases)):
        y_ref, _ = oracle.lora_forward(prob)
        assert np.array_equal(B.to_host_bits(c.y, "bf16"), f32_to_bf16_bits(y_ref.astype(np.float32))), p


def test_one_token_and_empty():
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    probs = projections(np.array([3], dtype=np.int32), [(256, 128, [8] * 4), (512, 64, [16] * 4)], "bf16", seed=81)
    say("case grouped one token")
    cases = run_grouped(probs)
    check_against_oracle(probs, cases, "one_token")
    say("case grouped empty batch")
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(0, dtype=torch.int32, device="cuda")
    projs = B.proj_array([x], [cases[0].pool], [y])
    B.bgmv_grouped([x], ids, [cases[0].pool], [y], torch.zeros(16, dtype=torch.uint8, device="cuda"), "bf16",
                   projs=projs)
    torch.cuda.synchronize()


def test_rejects_shared_output():
    from segmented_gather_gemm_lora_amd import binding as B

    probs = projections(np.array([0, 1, 0], dtype=np.int32), [(64, 32, [4, 8]), (64, 32, [4, 8])], "bf16", seed=91)
    cases = [GpuCase(p) for p in probs]
    xs, pools = [c.x for c in cases], [c.pool for c in cases]
    ys = [cases[0].y, cases[0].y]
    projs = B.proj_array(xs, pools, ys)
    ws = B.bgmv_grouped_workspace(3, projs)
    with pytest.raises(B.LoraError):
        B.bgmv_grouped(xs, cases[0].ids_dev, pools, ys, ws, "bf16", projs=projs)


def _qkv_small(seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, 24, 48).astype(np.int32)
    ids[rng.random(48) < 0.1] = -1
    specs = [(512, 512, [16] * 24), (512, 128, [8] * 24), (512, 128, [32] * 24)]
    return projections(ids, specs, "bf16", seed=seed, share_x=True)


def test_grouped_onepass_repeated_calls():
    """Eight calls in a row of the one-launch grouped form on one workspace,
    nothing reset in between: every call gives the same bits as a single
    lora_bgmv call of each projection, and the status word stays zero."""
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    probs = _qkv_small(101)
    cases = [GpuCase(p, y_init="zero") for p in probs]
    for c in cases[1:]:
        c.x = cases[0].x
    xs, pools, ys = [c.x for c in cases], [c.pool for c in cases], [c.y for c in cases]
    projs = B.proj_array(xs, pools, ys)
    ws = B.bgmv_grouped_workspace(probs[0].T, projs)
    singles = []
    for prob in probs:
        s = GpuCase(prob, y_init="zero")
        s.x = cases[0].x
        w1 = B.workspace(B.LORA_OP_BGMV, prob.T, prob.d_in, prob.d_out, prob.max_rank)
        B.bgmv(s.x, s.ids_dev, s.pool, s.y, w1, "bf16")
        torch.cuda.synchronize()
        singles.append(B.to_host_bits(s.y, "bf16"))
    say("case grouped one-launch repeated calls")
    for _ in range(8):
        for c in cases:
            c.y.zero_()
        B.bgmv_grouped(xs, cases[0].ids_dev, pools, ys, ws, "bf16", projs=projs)
        torch.cuda.synchronize()
        assert B.workspace_status(ws) == 0
        for p, c in enumerate(cases):
            assert np.array_equal(B.to_host_bits(c.y, "bf16"), singles[p]), f"proj{p} differs from lora_bgmv"


def test_grouped_onepass_forced_give_up_ends_normally():
    """The host forces every wait of the one-launch grouped kernel to give up
    at once: the kernel still ends, the status word is set and every y is left
    as it was.  The next call (default wait) is correct; lora_workspace_clear
    resets the status."""
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    probs = _qkv_small(102)
    cases = [GpuCase(p) for p in probs]
    for c in cases[1:]:
        c.x = cases[0].x
    xs, pools, ys = [c.x for c in cases], [c.pool for c in cases], [c.y for c in cases]
    before = [B.to_host_bits(c.y, "bf16") for c in cases]
    projs = B.proj_array(xs, pools, ys)
    ws = B.bgmv_grouped_workspace(probs[0].T, projs)
    say("case grouped one-launch forced give-up")
    B.debug_wait_limit(-1)
    try:
        B.bgmv_grouped(xs, cases[0].ids_dev, pools, ys, ws, "bf16", projs=projs)
        torch.cuda.synchronize()
    finally:
        B.debug_wait_limit(0)
    assert B.workspace_status(ws) == 1
    for p, c in enumerate(cases):
        assert np.array_equal(B.to_host_bits(c.y, "bf16"), before[p]), f"proj{p}: a consumer that gave up wrote y"
    say("case grouped one-launch after a give-up")
    B.bgmv_grouped(xs, cases[0].ids_dev, pools, ys, ws, "bf16", projs=projs)
    torch.cuda.synchronize()
    check_against_oracle(probs, cases, "after give-up")
    assert B.workspace_status(ws) == 1  # sticky until cleared
    B.workspace_clear(ws)
    torch.cuda.synchronize()
    assert B.workspace_status(ws) == 0
