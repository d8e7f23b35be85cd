"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerances (per element): fp32 |gpu - ref| <= 1e-5 (|ref| + 1); bf16 inputs
with fp32 accumulation |gpu - ref| <= 2e-2 (|ref| + 1e-2).  The shrink result v
is checked against the oracle's v with the rigorous fp32 summation bound
d_in * 2^-24 * sum_k |x_k A_jk|.  Each named workload runs as specified (y
preset) and with a zero base, so that the tolerance scales with the
correction itself.
"""

import numpy as np
import pytest

import oracle
from gpu_helpers import GpuCase, assert_close, decode, require_gpu, say, v_bound
from lora_workloads import make_config, make_integer_problem, make_problem

pytestmark = pytest.mark.gpu

_ORACLE_CACHE = {}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    oracle.build(force=False)
    return require_gpu()


def oracle_ref(key, prob, zero_base=False):
    if key not in _ORACLE_CACHE:
        p = prob
        if zero_base:
            p = _with_zero_base(prob)
        _ORACLE_CACHE[key] = oracle.lora_forward(p, want_v=True, nthreads=16)
    return _ORACLE_CACHE[key]


def _with_zero_base(prob):
    import copy

    q = copy.copy(prob)
    q.y_in = None
    return q


def check_case(prob, path, zero_base, key=None):
    say(f"case {prob.name} T={prob.T} d_in={prob.d_in} d_out={prob.d_out} dtype={prob.dtype} path={path} "
        f"zero_base={zero_base}")
    c = GpuCase(prob, y_init="zero" if zero_base else "stored")
    v, plan = c.run(path)
    y = c.y_out()
    y_ref, v_ref = oracle_ref(key, prob, zero_base) if key else oracle.lora_forward(
        _with_zero_base(prob) if zero_base else prob, want_v=True, nthreads=16)
    worst = assert_close(y, y_ref, prob.dtype, f"{prob.name}/{path}/y")
    none = np.nonzero(prob.ids < 0)[0]
    if len(none):  # rows of tokens without an adapter are untouched (bitwise)
        y0 = decode(c.y_host_in, prob.dtype)
        assert np.array_equal(y[none], y0[none])
    if v is None:
        return worst
    # v: rows in sorted order (SGMV) or token order (BGMV)
    if path == "sgmv_split":
        perm = plan.arrays()["perm"]
        vv, tok = v[: len(perm)], perm
    else:
        tok = np.nonzero(prob.ids >= 0)[0]
        vv = v[tok]
    ranks = prob.ranks[prob.ids[tok]] if len(tok) else np.zeros(0, dtype=np.int32)
    bound = v_bound(prob, tok, prob.ids[tok])
    for i, t in enumerate(tok):
        r = int(ranks[i])
        err = np.abs(vv[i, :r] - v_ref[t, :r])
        assert (err <= bound[i, :r] + 1e-6 * np.abs(v_ref[t, :r])).all(), (prob.name, path, "v", t)
    return worst


ALL_PATHS = ["sgmv", "bgmv", "sgmv_split", "bgmv_split"]


@pytest.mark.parametrize("zero_base", [False, True], ids=["y_preset", "y_zero"])
@pytest.mark.parametrize("path", ALL_PATHS)
@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_named_workloads(k, path, zero_base):
    prob = make_config(k)
    check_case(prob, path, zero_base, key=(k, zero_base))


@pytest.mark.parametrize("k,seed", [(2, 102), (3, 103), (4, 104)])
def test_named_workloads_other_seeds(k, seed):
    prob = make_config(k, seed=seed)
    check_case(prob, "sgmv" if k != 2 else "bgmv", False)
    check_case(prob, "sgmv_split" if k != 2 else "bgmv_split", False)


SHAPES = [
    # name, dtype, T, d_in, d_out, ranks, none_frac, seed
    ("ragged_d", "bf16", 53, 37, 29, [3, 1, 16, 7], 0.1, 1),
    ("ragged_d_f32", "f32", 41, 45, 301, [5, 8, 2], 0.2, 2),
    ("rank1", "bf16", 33, 256, 300, [1], 0.0, 3),
    ("rank256", "bf16", 40, 512, 520, [256, 200], 0.0, 4),
    ("rank256_f32", "f32", 19, 136, 264, [256, 33], 0.0, 5),
    ("one_token", "bf16", 1, 4096, 4096, [16], 0.0, 6),
    ("many_tiny_segments", "bf16", 300, 1024, 768, list(range(1, 65)), 0.05, 7),
    ("long_and_short", "bf16", 700, 2048, 1100, [64, 8, 32, 16], 0.0, 8),
    ("wide_out", "bf16", 24, 128, 14336, [8, 64], 0.0, 9),
]


@pytest.mark.parametrize("path", ALL_PATHS)
@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_shapes(shape, path):
    name, dt, T, d_in, d_out, ranks, none_frac, seed = shape
    rng = np.random.default_rng(seed)
    n = len(ranks)
    if name == "long_and_short":
        ids = np.concatenate([np.full(600, 0), rng.integers(1, n, T - 600)]).astype(np.int32)
    else:
        ids = rng.integers(0, n, T).astype(np.int32)
    ids[rng.random(T) < none_frac] = -1
    prob = make_problem(name=name, dtype=dt, ids=ids, ranks=ranks, alphas=[2.0 * r for r in ranks], d_in=d_in,
                        d_out=d_out, seed=seed, a_std=0.05, b_std=0.05)
    check_case(prob, path, False)
    check_case(prob, path, True)


LONG_SEGMENT_SHAPES = [
    # name, segment lengths, ranks, d_in, d_out, shuffled token order, none_frac, seed
    # d_in 4608 is split into 3 slices of 1536 (a ragged last 512 of each)
    ("mixed_lengths", [145, 40, 16, 130], [16, 5, 1, 13], 4608, 384, True, 0.05, 21),
    ("d_in_8192", [200, 300], [16, 8], 8192, 256, False, 0.0, 22),
    ("short_d_in", [100, 70], [12, 16], 200, 100, True, 0.0, 23),
    ("prefill_like", [900, 37, 1500, 611], [16, 16, 16, 16], 4096, 4096, False, 0.0, 24),
]


def segmented_problem(name, lens, ranks, d_in, d_out, shuffled, none_frac, seed):
    """Segments of the given lengths (adapter i for segment i), in token order,
    shuffled so that every segment's rows are gathered (True), or with only the
    tokens after the first segment shuffled ("tail")."""
    rng = np.random.default_rng(seed)
    ids = np.repeat(np.arange(len(lens), dtype=np.int32), lens)
    if shuffled == "tail":
        ids[lens[0]:] = rng.permutation(ids[lens[0]:])
    elif shuffled:
        ids = rng.permutation(ids).astype(np.int32)
    ids[rng.random(len(ids)) < none_frac] = -1
    return make_problem(name=name, dtype="bf16", ids=ids, ranks=ranks, alphas=[2.0 * r for r in ranks], d_in=d_in,
                        d_out=d_out, seed=seed, a_std=0.05, b_std=0.05)


@pytest.mark.parametrize("shape", LONG_SEGMENT_SHAPES, ids=[s[0] for s in LONG_SEGMENT_SHAPES])
def test_long_segment_shapes(shape):
    prob = segmented_problem(*shape)
    check_case(prob, "sgmv", False)
    check_case(prob, "sgmv", True)


def test_long_segment_integer_bitwise():
    """Entries in {-1,0,1}, scale 1, two long segments over d_in 4608 (three
    slices): fp32 sums are exact, so the bf16 output equals the exact integer
    result rounded once."""
    from lora_workloads import f32_to_bf16_bits
    from segmented_gather_gemm_lora_amd import binding as B

    prob = make_integer_problem(seed=31, dtype="bf16", T=300, d_in=4608, d_out=200, n_adapters=2, ranks=[3, 4],
                                none_frac=0.05)
    say("case long-segment integer")
    c = GpuCase(prob)
    c.run("sgmv")
    y_ref, _ = oracle.lora_forward(prob)
    assert np.array_equal(B.to_host_bits(c.y, "bf16"), f32_to_bf16_bits(y_ref.astype(np.float32)))


ARG_TABLE_CHUNKS = 112  # chunk descriptors the chunked expand takes in its kernel arguments


def chunked_expand(plan, d_out):
    """Whether the SGMV expand runs on 64-row chunks (chunks x 256-column tiles
    >= 1024 and max rank <= 32), and whether its chunk table fits in the kernel
    arguments."""
    h = plan.header()
    ncol = (d_out + 255) // 256
    return h["num_chunks"] * ncol >= 1024 and h["max_rank"] <= 32, h["num_chunks"] <= ARG_TABLE_CHUNKS


CHUNK_EXPAND_SHAPES = [
    # name, segment lengths, ranks, d_in, d_out, shuffled, none_frac, seed, expected table use
    # every chunk gathered (rows not consecutive)
    ("gathered_rows", [700, 500, 600, 248], [16, 8, 4, 12], 256, 8192, True, 0.0, 41, True),
    # consecutive chunks next to gathered ones, ranks up to 32 (two 16-rank steps)
    ("mixed_rows", [1100, 300, 300, 300], [32, 16, 24, 8], 256, 8192, "tail", 0.0, 42, True),
    # more chunks than the argument table holds: descriptors read from the plan
    ("table_overflow", [5000, 3000], [16, 8], 256, 4096, False, 0.02, 43, False),
]


@pytest.mark.parametrize("shape", CHUNK_EXPAND_SHAPES, ids=[s[0] for s in CHUNK_EXPAND_SHAPES])
def test_chunk_expand_shapes(shape):
    *args, table = shape
    prob = segmented_problem(*args)
    _, plan = GpuCase(prob).run("sgmv")
    assert chunked_expand(plan, prob.d_out) == (True, table), "shape no longer reaches the intended expand"
    check_case(prob, "sgmv", False)
    check_case(prob, "sgmv_split", True)


@pytest.mark.parametrize("path", ALL_PATHS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_tokens_without_adapter(dtype, path):
    prob = make_problem(name="none", dtype=dtype, ids=[-1] * 20, ranks=[4, 8], alphas=[1.0, 1.0], d_in=64, d_out=48,
                        seed=1)
    say(f"case all-none {dtype} {path}")
    c = GpuCase(prob)
    c.run(path)
    assert np.array_equal(B_bits(c), prob.y_in)


def B_bits(c):
    from segmented_gather_gemm_lora_amd import binding as B

    return B.to_host_bits(c.y, c.dt)


@pytest.mark.parametrize("path", ["sgmv", "bgmv"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_empty_batch(dtype, path):
    """T = 0 is a successful no-op on both paths."""
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    prob = make_problem(name="empty", dtype=dtype, ids=np.zeros(0, dtype=np.int32), ranks=[4], alphas=[1.0], d_in=64,
                        d_out=48, seed=1)
    pool = B.DevicePool.from_problem(prob)
    say(f"case empty {dtype} {path}")
    x = torch.zeros((0, 64), dtype=B.torch_dtype(dtype), device="cuda")
    y = torch.zeros((0, 48), dtype=B.torch_dtype(dtype), device="cuda")
    v = torch.zeros((1, 4), device="cuda")
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    if path == "sgmv":
        plan = B.Plan(1).build(prob.ids, pool).upload()
        assert plan.header()["num_sorted"] == 0
        B.sgmv_shrink(x, plan, v, dtype)
        B.sgmv_expand(v, plan, y, dtype)
        B.sgmv(x, plan, y, ws, dtype)
    else:
        ids = torch.zeros(0, dtype=torch.int32, device="cuda")
        B.bgmv_shrink(x, ids, pool, v, dtype)
        B.bgmv_expand(v, ids, pool, y, dtype)
        B.bgmv(x, ids, pool, y, ws, dtype)
    torch.cuda.synchronize()


@pytest.mark.parametrize("path", ALL_PATHS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_integer_bitwise(seed, dtype, path):
    """Entries in {-1,0,1}, scale 1: every partial sum is a small integer, so
    the GPU must reproduce the oracle exactly (bitwise)."""
    prob = make_integer_problem(seed=seed, dtype=dtype, T=40, d_in=16, d_out=16, n_adapters=3, none_frac=0.1)
    say(f"case integer seed={seed} {dtype} {path}")
    c = GpuCase(prob)
    c.run(path)
    y = c.y_out()
    y_ref, _ = oracle.lora_forward(prob)
    assert np.array_equal(y, y_ref)


@pytest.mark.parametrize("path", ALL_PATHS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_integer_bitwise_larger(dtype, path):
    """Larger integer case (d_in 200, ranks 1..4, d_out 333): fp32 sums are
    exact; a bf16 output equals the exact integer rounded once to bf16."""
    from lora_workloads import f32_to_bf16_bits

    prob = make_integer_problem(seed=11, dtype=dtype, T=70, d_in=200, d_out=333, n_adapters=5, none_frac=0.1)
    say(f"case integer-larger {dtype} {path}")
    c = GpuCase(prob)
    c.run(path)
    y_ref, _ = oracle.lora_forward(prob)
    from segmented_gather_gemm_lora_amd import binding as B

    bits = B.to_host_bits(c.y, dtype)
    if dtype == "bf16":
        assert np.array_equal(bits, f32_to_bf16_bits(y_ref.astype(np.float32)))
    else:
        assert np.array_equal(bits, y_ref.astype(np.float32))


@pytest.mark.parametrize("path", ["bgmv", "bgmv_split"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,n_pool", [(8, 50), (40, 200), (3, 1000)])
def test_bgmv_large_pool(T, n_pool, dtype, path):
    """Pools larger than twice the batch take the leader-token grid (one
    workgroup per token; the first token of each adapter serves its group)."""
    rng = np.random.default_rng(T * 7 + n_pool)
    ranks = rng.choice([4, 8, 16, 24], n_pool).tolist()
    ids = rng.integers(0, min(n_pool, 6), T).astype(np.int32)  # repeats: groups of several tokens
    ids[rng.random(T) < 0.2] = -1
    prob = make_problem(name=f"pool{n_pool}", dtype=dtype, ids=ids, ranks=ranks, alphas=[2.0 * r for r in ranks],
                        d_in=256, d_out=320, seed=T + n_pool, a_std=0.05, b_std=0.05)
    check_case(prob, path, False)
    check_case(prob, path, True)


def test_segments_boundary_end_to_end():
    """The batch's segments through the boundary calls alone: lora_segments_bind
    on a pinned host buffer and a device buffer, lora_build_segments,
    lora_segments_upload, then lora_sgmv.  The device copy of the segment table
    equals the host one (and the oracle's brute-force segments), and y matches
    the oracle."""
    import ctypes

    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    prob = make_config(4)  # mixed ranks, Zipf ids, decode tokens and long segments
    say("case segments boundary end to end")
    pool = B.DevicePool.from_problem(prob)
    T = prob.T
    nbytes = B.lora_segments_bytes(T)
    hbuf = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dbuf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    hs, ds = B.LoraSegments(), B.LoraSegments()
    assert B.lora_segments_bind(hbuf.data_ptr(), T, ctypes.addressof(hs)) == 0
    assert B.lora_segments_bind(dbuf.data_ptr(), T, ctypes.addressof(ds)) == 0
    ids = np.ascontiguousarray(prob.ids, dtype=np.int32)
    assert B.lora_build_segments(T, ids.ctypes.data, pool.n_adapters, pool.addr_A.ctypes.data,
                                 pool.addr_B.ctypes.data, pool.rank.ctypes.data, pool.alpha.ctypes.data,
                                 ctypes.addressof(hs)) == 0, B.last_error()
    stream = torch.cuda.current_stream()
    assert B.lora_segments_upload(ctypes.addressof(hs), ctypes.addressof(ds), stream.cuda_stream) == 0
    torch.cuda.synchronize()
    assert (ds.num_segments, ds.num_tokens, ds.max_rank) == (hs.num_segments, hs.num_tokens, hs.max_rank)
    assert ds.host == hbuf.data_ptr() and ds.buf == dbuf.data_ptr()
    # the device struct's arrays, read back through their device addresses
    dev = dbuf.cpu().numpy()
    base = dbuf.data_ptr()
    S, Tp = ds.num_segments, ds.num_tokens

    def read(addr, dtype, n):
        off = addr - base
        return dev[off: off + n * np.dtype(dtype).itemsize].view(dtype)

    host = B.segment_table(hs)
    perm_o, indptr_o, adapter_o = oracle.segments(prob.ids, prob.n_adapters)
    assert np.array_equal(read(ds.perm, np.int32, Tp), perm_o) and np.array_equal(host["perm"], perm_o)
    assert np.array_equal(read(ds.seg_indptr, np.int32, S + 1), indptr_o)
    assert np.array_equal(read(ds.seg_adapter, np.int32, S), adapter_o)
    assert np.array_equal(read(ds.seg_rank, np.int32, S), prob.ranks[adapter_o])
    assert np.array_equal(read(ds.seg_A, np.uint64, S), pool.addr_A[adapter_o])
    assert np.array_equal(read(ds.seg_B, np.uint64, S), pool.addr_B[adapter_o])
    assert np.array_equal(read(ds.seg_scale, np.float32, S), host["seg_scale"])
    c = GpuCase(prob, y_init="zero")
    ws = B.workspace(B.LORA_OP_SGMV, T, prob.d_in, prob.d_out, prob.max_rank)
    assert B.lora_sgmv(stream.cuda_stream, B.LORA_BF16, c.x.data_ptr(), c.x.stride(0), prob.d_in,
                       ctypes.addressof(ds), c.y.data_ptr(), c.y.stride(0), prob.d_out, ws.data_ptr(),
                       ws.numel()) == 0, B.last_error()
    torch.cuda.synchronize()
    y_ref, _ = oracle.lora_forward(_with_zero_base(prob), nthreads=16)
    assert_close(c.y_out(), y_ref, "bf16", "segments boundary")


def test_per_chunk_form_choice_in_one_launch():
    """One expand launch over a plan mixing long segments (64-row chunk form;
    ranks <= 32 with B held, 33 .. 64 with B packed) and short ones (16-row
    block form), ranks not a multiple of 4 included (block form for every
    chunk): lora_sgmv enqueues the shrink and one expand, and y matches the
    oracle."""
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    rng = np.random.default_rng(77)
    ranks = [64, 48, 40, 8, 33, 16, 32, 1, 64, 12]
    long_ids = np.repeat(np.arange(5), [300, 130, 70, 200, 90])      # long segments, ranks 64, 48, 40, 8, 33
    short_ids = rng.integers(5, 10, 60)                                # short ones over the other adapters
    ids = np.concatenate([long_ids, short_ids]).astype(np.int32)
    ids = ids[rng.permutation(len(ids))]
    ids[rng.random(len(ids)) < 0.03] = -1
    prob = make_problem(name="mixed_forms", dtype="bf16", ids=ids, ranks=ranks, alphas=[32.0] * len(ranks),
                        d_in=1024, d_out=2560, seed=77, a_std=0.05, b_std=0.05)
    say("case per-chunk form choice in one launch")
    c = GpuCase(prob, y_init="zero")
    timer = B.KernelTimer(8)
    timer.arm(0, 8)
    c.run("sgmv")
    assert B.KernelTimer.used() == 2, "shrink + one expand"
    timer.disarm()
    timer.close()
    torch.cuda.synchronize()
    y_ref, _ = oracle.lora_forward(_with_zero_base(prob), nthreads=16)
    assert_close(c.y_out(), y_ref, "bf16", "mixed forms")
    # the same batch, y preset
    c2 = GpuCase(prob)
    c2.run("sgmv")
    y_ref2, _ = oracle.lora_forward(prob, nthreads=16)
    assert_close(c2.y_out(), y_ref2, "bf16", "mixed forms, y preset")
