"""Grouped SGMV (prefill form of the grouped invocation, "Multi-LoRA Serving
in Production ..." (llms.blog), section "Ragged Batching and FlashInfer
Grouped GEMM"): several projections of a layer, each with its own plan (the
batch's ids with the projection's own adapters), x, y and sizes, in one
shrink and one expand launch.

Each projection is checked against the fp64 oracle of that projection alone
(bf16 |gpu - ref| <= 2e-2 (|ref| + 1e-2); fp32 <= 1e-5 (|ref| + 1)), and
bitwise against a single lora_sgmv call of that projection where the single
call takes the same kernel variants (16-row block expand).
"""

import copy

import numpy as np
import pytest

import oracle
from gpu_helpers import assert_close, decode, require_gpu, say
from lora_workloads import make_config, make_problem

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    oracle.build(force=False)
    return require_gpu()


def mixed_ids(T, n_adapters, seed):
    """Long and short segments, shuffled, and tokens without an adapter."""
    rng = np.random.default_rng(seed)
    ids = []
    while len(ids) < T:
        ids += [int(rng.integers(0, n_adapters))] * int(rng.choice([1, 2, 5, 17, 40, 130]))
    ids = np.array(ids[:T], dtype=np.int32)
    ids[rng.random(T) < 0.05] = -1
    return ids


def projections(ids, dtype, d_ins, d_outs, ranks_of, seed, shared_x=True):
    probs = []
    for p, (d_in, d_out) in enumerate(zip(d_ins, d_outs)):
        ranks = ranks_of(p)
        q = make_problem(name=f"grouped_sgmv_p{p}", dtype=dtype, ids=ids, ranks=ranks,
                         alphas=[2.0 * r for r in ranks], d_in=d_in, d_out=d_out, seed=seed + p, a_std=0.05,
                         b_std=0.05)
        if shared_x and p > 0:
            q = copy.copy(q)
            q.x = probs[0].x
        probs.append(q)
    return probs


def run_grouped(probs, zero_base, plans_override=None):
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    dt = probs[0].dtype
    pools = [B.DevicePool.from_problem(q) for q in probs]
    plans = plans_override or [B.Plan(q.T).build(q.ids, pool).upload() for q, pool in zip(probs, pools)]
    xs, ys, y0 = [], [], []
    x_shared = None
    for p, q in enumerate(probs):
        if p > 0 and q.x is probs[0].x:
            xs.append(x_shared)
        else:
            x_shared = B.to_device(q.x, dt)
            xs.append(x_shared)
        yin = np.zeros((q.T, q.d_out), dtype=np.uint16 if dt == "bf16" else np.float32) if zero_base else q.y_base()
        y0.append(yin)
        ys.append(B.to_device(yin, dt))
    ws = B.sgmv_grouped_workspace(plans, xs, ys)
    timer = B.KernelTimer(8)
    timer.arm(0, 8)
    B.sgmv_grouped(xs, plans, ys, ws, dt)
    used = B.KernelTimer.used()
    timer.disarm()
    timer.close()
    torch.cuda.synchronize()
    return [B.to_host_bits(y, dt) for y in ys], y0, xs, pools, plans, used


def single_call(q, x, pool, plan, yin):
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    y = B.to_device(yin, q.dtype)
    ws = B.workspace(B.LORA_OP_SGMV, q.T, q.d_in, q.d_out, max(q.max_rank, 1))
    B.sgmv(x, plan, y, ws, q.dtype)
    torch.cuda.synchronize()
    return B.to_host_bits(y, q.dtype)


def check(probs, zero_base, bitwise=True):
    outs, y0, xs, pools, plans, used = run_grouped(probs, zero_base)
    assert used == 2, f"{used} launches"
    for p, q in enumerate(probs):
        ref_p = copy.copy(q)
        if zero_base:
            ref_p.y_in = None
        ref, _ = oracle.lora_forward(ref_p, nthreads=16)
        assert_close(decode(outs[p], q.dtype), ref, q.dtype, f"projection {p}")
        none = np.nonzero(q.ids < 0)[0]
        assert np.array_equal(outs[p][none], y0[p][none])
        if bitwise:
            h = plans[p].header()
            ncol = (q.d_out + 255) // 256
            assert h["num_chunks"] * ncol < 1024 or h["max_rank"] > 32, "single call would take the chunk expand"
            assert np.array_equal(outs[p], single_call(q, xs[p], pools[p], plans[p], y0[p])), f"projection {p}"


@pytest.mark.parametrize("zero_base", [True, False], ids=["y_zero", "y_preset"])
def test_grouped_sgmv_qkv_bf16(zero_base):
    """q, k, v of one layer: shared x (1024 wide), d_out 1024 / 256 / 256, own
    adapters per projection with mixed ranks, ragged segments."""
    say(f"case grouped sgmv qkv bf16 zero_base={zero_base}")
    ids = mixed_ids(700, 6, seed=21)
    ranks = {0: [16, 8, 32, 16, 4, 12], 1: [8, 8, 16, 5, 8, 8], 2: [16, 1, 16, 16, 3, 16]}
    check(projections(ids, "bf16", [1024] * 3, [1024, 256, 256], lambda p: ranks[p], seed=30), zero_base)


def test_grouped_sgmv_own_inputs_f32():
    """Projections with their own x and different d_in (one not a multiple of 8:
    scalar loads for all), fp32."""
    say("case grouped sgmv own inputs f32")
    ids = mixed_ids(300, 4, seed=5)
    probs = projections(ids, "f32", [512, 300, 768], [384, 520, 64], lambda p: [8, 16, 4, 7][: 4], seed=40,
                        shared_x=False)
    check(probs, zero_base=False)


def test_grouped_sgmv_skips_empty_projection():
    """A projection whose plan has no adapted token is skipped; the others run."""
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    say("case grouped sgmv empty projection")
    ids = mixed_ids(200, 3, seed=9)
    probs = projections(ids, "bf16", [256, 256], [256, 512], lambda p: [8, 16, 8], seed=50)
    pools = [B.DevicePool.from_problem(q) for q in probs]
    none_ids = np.full(200, -1, dtype=np.int32)
    plans = [B.Plan(200).build(probs[0].ids, pools[0]).upload(), B.Plan(200).build(none_ids, pools[1]).upload()]
    outs, y0, *_ = run_grouped(probs, zero_base=False, plans_override=plans)
    assert np.array_equal(outs[1], y0[1])
    ref, _ = oracle.lora_forward(probs[0], nthreads=16)
    assert_close(decode(outs[0], "bf16"), ref, "bf16", "projection 0")


def test_grouped_sgmv_prefill_qkv():
    """The prefill workload's segments (4096 tokens, 16 Dirichlet segments) as
    q, k, v: d_out 4096 / 1024 / 1024, rank 16, against the oracle."""
    say("case grouped sgmv prefill qkv")
    base = make_config(3)
    probs = projections(base.ids, "bf16", [4096] * 3, [4096, 1024, 1024], lambda p: [16] * base.n_adapters,
                        seed=60)
    outs, y0, *_ , used = run_grouped(probs, zero_base=True)
    assert used == 2
    for p, q in enumerate(probs):
        r = copy.copy(q)
        r.y_in = None
        ref, _ = oracle.lora_forward(r, nthreads=16)
        assert_close(decode(outs[p], "bf16"), ref, "bf16", f"prefill projection {p}")


def test_grouped_sgmv_chunk_expand_rank32():
    """Enough (chunk, column tile) items for the 64-row chunk expand, ranks up
    to 32 (two 16-rank steps) including ranks that are not multiples of 4
    (scalar B loads), d_out 4096 / 1024 / 1024, against the oracle."""
    say("case grouped sgmv chunk expand rank 32")
    rng = np.random.default_rng(77)
    ids = np.repeat(rng.permutation(12), 256).astype(np.int32)
    ids[rng.random(ids.size) < 0.03] = -1
    ranks = {0: [32, 24, 17, 32, 8, 16, 32, 30, 32, 9, 20, 32], 1: [16, 32, 8, 5, 32, 16, 12, 32, 32, 32, 4, 28],
             2: [32] * 12}
    probs = projections(ids, "bf16", [1024] * 3, [4096, 1024, 1024], lambda p: ranks[p], seed=80)
    from segmented_gather_gemm_lora_amd import binding as B

    pools = [B.DevicePool.from_problem(q) for q in probs]
    plans = [B.Plan(q.T).build(q.ids, pool).upload() for q, pool in zip(probs, pools)]
    items = sum(pl.header()["num_chunks"] * ((q.d_out + 255) // 256) for pl, q in zip(plans, probs))
    assert items >= 1024, items
    outs, y0, *_, used = run_grouped(probs, zero_base=True, plans_override=plans)
    assert used == 2
    for p, q in enumerate(probs):
        r = copy.copy(q)
        r.y_in = None
        ref, _ = oracle.lora_forward(r, nthreads=16)
        assert_close(decode(outs[p], "bf16"), ref, "bf16", f"projection {p}")
