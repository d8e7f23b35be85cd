"""The adapter residency cache on the GPU: adapters registered from pinned host
memory are copied into a cache that holds only a few of them, on a copy stream,
and batch after batch runs on the compute stream with the cache's tables
(SGMV through a plan built from the host mirrors, BGMV through the device
tables).  Batches are enqueued back to back without host synchronisation, so
a copy that overwrote an adapter a running batch still reads, or a batch that
ran before its adapters arrived, would show in the results.  Every batch's
output is compared with the fp64 oracle of that batch (tolerance as for the
other bf16 paths: |gpu - ref| <= 2e-2 (|ref| + 1e-2))."""

import dataclasses

import numpy as np
import pytest

import oracle
from gpu_helpers import assert_close, decode, require_gpu, say
from lora_workloads import make_problem

pytestmark = pytest.mark.gpu

D_IN, D_OUT = 512, 384


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    oracle.build(force=False)
    return require_gpu()


def up(v):
    return (v + 255) // 256 * 256


def setup_cache(ranks, cache_units, seed, pageable=()):
    """A master problem holding every adapter, pinned host copies of each (plain
    pageable numpy arrays for the adapters in `pageable`, which the cache copies
    with hipMemcpyAsync instead of its copy kernel), and a cache with room for
    about `cache_units` adapters of the largest rank."""
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    n = len(ranks)
    master = make_problem(name="residency", dtype="bf16", ids=[0], ranks=ranks, alphas=[2.0 * r for r in ranks],
                          d_in=D_IN, d_out=D_OUT, seed=seed, a_std=0.05, b_std=0.05)
    rmax = max(ranks)
    nbytes = B.load().lora_cache_table_bytes(n) + cache_units * (up(rmax * D_IN * 2) + up(D_OUT * rmax * 2))
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    cache = B.AdapterCache(buf, n, "bf16", D_IN, D_OUT)
    for a, r in enumerate(ranks):
        A = master.pool[master.a_off[a]: master.a_off[a] + r * D_IN].copy()
        Bm = master.pool[master.b_off[a]: master.b_off[a] + D_OUT * r].copy()
        if a not in pageable:
            A, Bm = torch.from_numpy(A).pin_memory(), torch.from_numpy(Bm).pin_memory()
        cache.register(a, A, Bm, r, float(master.alphas[a]))
    return master, cache


def batch_problem(master, ids, seed):
    rng = np.random.default_rng(seed)
    T = len(ids)
    from lora_workloads import f32_to_bf16_bits

    x = f32_to_bf16_bits(rng.standard_normal((T, D_IN), dtype=np.float32))
    y = f32_to_bf16_bits(rng.standard_normal((T, D_OUT), dtype=np.float32))
    return dataclasses.replace(master, T=T, ids=np.asarray(ids, dtype=np.int32), x=x, y_in=y)


@pytest.mark.parametrize("path", ["sgmv", "bgmv"])
def test_batches_through_a_small_cache(path):
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    ranks = [8, 16, 32, 4, 16, 64, 8, 16, 32, 12, 16, 24]
    master, cache = setup_cache(ranks, cache_units=3, seed=7, pageable=(3, 9))
    copy_stream = torch.cuda.Stream()
    compute = torch.cuda.current_stream()
    rng = np.random.default_rng(11)
    runs = []
    for b in range(14):
        # each batch draws from 3 adapters, so consecutive batches evict each other's
        chosen = rng.choice(len(ranks), 3, replace=False)
        T = int(rng.integers(20, 90)) if path == "sgmv" else 48
        ids = rng.choice(chosen, T).astype(np.int32)
        ids[rng.random(T) < 0.1] = -1
        prob = batch_problem(master, ids, seed=100 + b)
        say(f"case residency {path} batch {b} adapters {sorted(set(ids[ids >= 0].tolist()))}")
        cache.prepare(ids, copy_stream, compute)
        pool = cache.pool()
        x = B.to_device(prob.x, "bf16")
        y = B.to_device(prob.y_in, "bf16")
        if path == "sgmv":
            plan = B.Plan(T).build(ids, pool).upload()
            ws = B.workspace(B.LORA_OP_SGMV, T, D_IN, D_OUT, max(ranks))
            B.sgmv(x, plan, y, ws, "bf16")
            keep = (plan, ws)
        else:
            ids_dev = torch.from_numpy(ids).cuda()
            ws = B.workspace(B.LORA_OP_BGMV, T, D_IN, D_OUT, max(ranks))
            B.bgmv(x, ids_dev, pool, y, ws, "bf16", max_rank=max(ranks))
            keep = (ids_dev, ws)
        runs.append((prob, y, keep))
    torch.cuda.synchronize()
    st = cache.stats()
    assert st["evictions"] > 0 and st["hits"] > 0 and st["batches"] == 14
    for b, (prob, y, _) in enumerate(runs):
        y_ref, _ = oracle.lora_forward(prob)
        got = decode(B.to_host_bits(y, "bf16"), "bf16")
        assert_close(got, y_ref, "bf16", f"batch {b}")
        none = np.nonzero(prob.ids < 0)[0]
        assert np.array_equal(got[none], decode(prob.y_in, "bf16")[none])
    cache.close()


def test_pinned_adapter_is_not_reloaded():
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    ranks = [16] * 6
    master, cache = setup_cache(ranks, cache_units=3, seed=8)
    cache.pin(0)
    copy_stream = torch.cuda.Stream()
    addr0 = None
    for b, pair in enumerate([(0, 1), (2, 3), (0, 4), (5, 2), (0, 1)]):
        ids = np.array([pair[0], pair[1]] * 8, dtype=np.int32)
        prob = batch_problem(master, ids, seed=200 + b)
        cache.prepare(ids, copy_stream, torch.cuda.current_stream())
        pool = cache.pool()
        addr0 = pool.addr_A[0] if addr0 is None else addr0
        assert pool.addr_A[0] == addr0, "the pinned adapter moved"
        plan = B.Plan(len(ids)).build(ids, pool).upload()
        x, y = B.to_device(prob.x, "bf16"), B.to_device(prob.y_in, "bf16")
        B.sgmv(x, plan, y, B.workspace(B.LORA_OP_SGMV, len(ids), D_IN, D_OUT, 16), "bf16")
        torch.cuda.synchronize()
        y_ref, _ = oracle.lora_forward(prob)
        assert_close(decode(B.to_host_bits(y, "bf16"), "bf16"), y_ref, "bf16", f"pinned batch {b}")
    st = cache.stats()
    # three slots, one pinned: adapter 0 is copied once and hit twice; the two
    # other slots take 1, 2, 3, 4, 5, 2, 1 in turn (least recently used out)
    assert (st["misses"], st["hits"], st["evictions"]) == (8, 2, 5)
    cache.close()
