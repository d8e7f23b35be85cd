"""Parity of the fused layer entry (y = x W0 + scale (x A) B, overwriting y)
with the fp64 oracle, through the C ABI.

bf16 tolerance as for the other paths: |gpu - ref| <= 2e-2 (|ref| + 1e-2).
Besides the layer as specified, every case also runs with W0 = 0, so that the
tolerance scales with the correction itself rather than with the base product.
The full-size fused workload (1024 tokens, 4096 -> 12288) is compared on every
output element.
"""

import copy

import numpy as np
import pytest

import oracle
from gpu_helpers import assert_close, decode, require_gpu, say
from lora_workloads import f32_to_bf16_bits, make_config, make_integer_problem, make_problem

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    oracle.build(force=False)
    return require_gpu()


def run_fused(prob, W0=None, pitch_pad=0):
    """Run lora_fused_linear on `prob` and return the output rows (float64).
    y gets a row pitch of round8(d_out) + pitch_pad elements."""
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    W0 = prob.W0 if W0 is None else W0
    pool = B.DevicePool.from_problem(prob)
    x = B.to_device(prob.x, "bf16")
    w = B.to_device(W0, "bf16")
    ldy = (prob.d_out + 7) // 8 * 8 + pitch_pad
    ybuf = torch.full((max(prob.T, 1), ldy), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = ybuf[: prob.T, : prob.d_out]
    plan = B.Plan(max(prob.T, 1)).build(prob.ids, pool).upload()
    ws = B.workspace(B.LORA_OP_FUSED, max(prob.T, 1), prob.d_in, prob.d_out, max(prob.max_rank, 1))
    B.fused_linear(x, w, plan, y, ws, "bf16")
    torch.cuda.synchronize()
    bits = y.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    pad = ybuf[: prob.T, prob.d_out:].float().cpu().numpy()
    assert np.isnan(pad).all(), "fused entry wrote outside the output rows"
    return bits


def oracle_rows(prob, rows, W0=None):
    sub = copy.copy(prob)
    rows = np.asarray(rows, dtype=np.int64)
    sub.T = len(rows)
    sub.ids = np.ascontiguousarray(prob.ids[rows])
    sub.x = np.ascontiguousarray(prob.x[rows])
    sub.y_in = None
    sub.W0 = prob.W0 if W0 is None else W0
    y, _ = oracle.lora_forward(sub, nthreads=16, fused=True)
    return y


def zero_w0(prob):
    return np.zeros_like(prob.W0)


@pytest.mark.parametrize("seed", [1, 2])
def test_fused_integer_bitwise(seed):
    """Entries in {-1,0,1}, scale 1: the fp32 sums are exact integers, so the
    bf16 output equals the exact result rounded once."""
    prob = make_integer_problem(seed=seed, dtype="bf16", T=300, d_in=200, d_out=333, n_adapters=5, none_frac=0.1,
                                with_w0=True)
    say(f"case fused integer seed={seed}")
    bits = run_fused(prob, pitch_pad=8)
    y_ref, _ = oracle.lora_forward(prob, fused=True)
    assert np.array_equal(bits, f32_to_bf16_bits(y_ref.astype(np.float32)))


SHAPES = [
    # name, T, d_in, d_out, ranks, none_frac, seed
    ("small_ragged", 37, 64, 40, [8, 16], 0.2, 1),
    ("tail_k_and_cols", 300, 200, 333, [8, 16, 32, 64], 0.1, 2),
    ("odd_ranks", 260, 136, 200, [5, 12, 1, 33], 0.05, 3),
    ("rank256", 96, 512, 392, [256, 100], 0.0, 4),
    ("many_segments", 520, 256, 584, list(range(1, 41)), 0.05, 5),
    ("all_none", 70, 64, 96, [4], 1.0, 6),
    ("one_token", 1, 128, 192, [16], 0.0, 7),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_fused_shapes(shape):
    name, T, d_in, d_out, ranks, none_frac, seed = shape
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, len(ranks), T).astype(np.int32)
    ids[rng.random(T) < none_frac] = -1
    prob = make_problem(name=name, dtype="bf16", ids=ids, ranks=ranks, alphas=[2.0 * r for r in ranks], d_in=d_in,
                        d_out=d_out, seed=seed, a_std=0.05, b_std=0.05, w0_std=0.05)
    say(f"case fused {name} T={T} d_in={d_in} d_out={d_out}")
    bits = run_fused(prob)
    y_ref, _ = oracle.lora_forward(prob, fused=True, nthreads=16)
    assert_close(decode(bits, "bf16"), y_ref, "bf16", f"fused {name}")
    say(f"case fused {name} W0=0")
    bits0 = run_fused(prob, W0=zero_w0(prob))
    y0, _ = oracle.lora_forward(_with_w0(prob, zero_w0(prob)), fused=True, nthreads=16)
    assert_close(decode(bits0, "bf16"), y0, "bf16", f"fused {name} W0=0")
    if (prob.ids < 0).any():
        assert (decode(bits0, "bf16")[prob.ids < 0] == 0).all()


def _with_w0(prob, W0):
    q = copy.copy(prob)
    q.W0 = W0
    return q


def test_fused_full_size_all_rows():
    """The full-size fused workload, every one of its 1024 x 12288 outputs
    compared with the oracle element by element, with W0 as drawn and with
    W0 = 0 (the tolerance then scales with the correction alone)."""
    prob = make_config(5)
    rows = np.arange(prob.T, dtype=np.int64)
    say(f"case fused full-size T={prob.T} d_in={prob.d_in} d_out={prob.d_out}")
    bits = run_fused(prob)
    y_ref = oracle_rows(prob, rows)
    assert_close(decode(bits, "bf16"), y_ref, "bf16", "fused full-size")
    say("case fused full-size W0=0")
    W0z = zero_w0(prob)
    bits0 = run_fused(prob, W0=W0z)
    y0 = oracle_rows(prob, rows, W0=W0z)
    assert_close(decode(bits0, "bf16"), y0, "bf16", "fused full-size W0=0")
    assert (decode(bits0, "bf16")[prob.ids < 0] == 0).all()


def test_fused_equals_base_plus_sgmv():
    """The fused call and the two-step path (base product stored as bf16,
    then an SGMV accumulate of the same plan) each match the oracle of what
    they compute: the fused layer, and the SGMV over the stored base."""
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    rng = np.random.default_rng(11)
    ranks = [8, 16, 64]
    ids = rng.integers(-1, 3, 400).astype(np.int32)
    prob = make_problem(name="fused_vs_sgmv", dtype="bf16", ids=ids, ranks=ranks, alphas=[32.0] * 3, d_in=256,
                        d_out=384, seed=11, a_std=0.05, b_std=0.05, w0_std=0.05)
    say("case fused vs base + sgmv")
    fused = decode(run_fused(prob), "bf16")
    # base through the fused entry with every token unadapted, then SGMV accumulate
    none = copy.copy(prob)
    none.ids = np.full_like(prob.ids, -1)
    base_bits = run_fused(none)
    pool = B.DevicePool.from_problem(prob)
    y = B.to_device(base_bits, "bf16")
    x = B.to_device(prob.x, "bf16")
    plan = B.Plan(prob.T).build(prob.ids, pool).upload()
    ws = B.workspace(B.LORA_OP_SGMV, prob.T, prob.d_in, prob.d_out, max(ranks))
    B.sgmv(x, plan, y, ws, "bf16")
    torch.cuda.synchronize()
    two_step = decode(B.to_host_bits(y, "bf16"), "bf16")
    y_ref, _ = oracle.lora_forward(prob, fused=True)
    assert_close(fused, y_ref, "bf16", "fused")
    stored = copy.copy(prob)
    stored.y_in = base_bits
    y_two, _ = oracle.lora_forward(stored, fused=False)
    assert_close(two_step, y_two, "bf16", "base + sgmv")
    base_ref, _ = oracle.lora_forward(none, fused=True)
    assert_close(decode(base_bits, "bf16"), base_ref, "bf16", "base only")


def test_fused_rejects_bad_arguments():
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    prob = make_problem(name="bad", dtype="bf16", ids=[0, 0, 1], ranks=[4, 8], alphas=[1.0, 1.0], d_in=64,
                        d_out=48, seed=1, w0_std=0.05)
    pool = B.DevicePool.from_problem(prob)
    x = B.to_device(prob.x, "bf16")
    w = B.to_device(prob.W0, "bf16")
    y = torch.zeros((3, 48), dtype=torch.bfloat16, device="cuda")
    plan = B.Plan(3).build(prob.ids, pool).upload()
    small = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.LoraError):
        B.fused_linear(x, w, plan, y, small, "bf16")  # workspace too small
    ws = B.workspace(B.LORA_OP_FUSED, 3, 64, 48, 8)
    with pytest.raises(B.LoraError):
        B.fused_linear(x[:, 1:], w, plan, y, ws, "bf16")  # misaligned rows
    torch.cuda.synchronize()
