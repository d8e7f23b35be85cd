"""Parity of the fused layer over an FP8 base (lora_fused_linear_e4m3: W0 holds
OCP E4M3 codes standing for w0_scale * code; x, y and the adapters bf16) with
the fp64 oracle, through the C ABI.

* every finite code, decoded by the kernel, gives exactly the oracle's value
  (one-hot x, power-of-two scale: the products are exact in bf16);
* a NaN code spreads to its output column only, as in the oracle;
* reduced shapes (ragged tails in tokens and columns, a half stage of k,
  ranks that are not multiples of 8, all tokens without an adapter), with
  the codes as drawn and with all codes zero (the tolerance then scales
  with the correction alone, which the kernel carries divided by w0_scale);
* the full-size workload (1024 tokens, 4096 -> 12288), every output element.

Tolerance: the bf16 bar of the other paths, |gpu - ref| <= 2e-2 (|ref| + 1e-2).
"""

import copy

import numpy as np
import pytest

import oracle
from gpu_helpers import assert_close, decode, require_gpu, say
from lora_workloads import f32_to_bf16_bits, make_fused_fp8, make_problem, with_e4m3_base

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    oracle.build(force=False)
    return require_gpu()


def run_fused_e4m3(prob, codes=None, scale=None, ids=None):
    """Run lora_fused_linear_e4m3 on `prob` (its E4M3 base unless `codes` is
    given) and return the output bits [T, d_out]."""
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    codes = prob.W0_e4m3 if codes is None else codes
    scale = prob.w0_scale if scale is None else scale
    ids = prob.ids if ids is None else ids
    pool = B.DevicePool.from_problem(prob)
    x = B.to_device(prob.x, "bf16")
    w = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).cuda()
    ldy = (prob.d_out + 7) // 8 * 8
    ybuf = torch.full((max(prob.T, 1), ldy), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = ybuf[: prob.T, : prob.d_out]
    plan = B.Plan(max(prob.T, 1)).build(ids, pool).upload()
    ws = B.workspace(B.LORA_OP_FUSED, max(prob.T, 1), prob.d_in, prob.d_out, max(prob.max_rank, 1))
    B.fused_linear_e4m3(x, w, scale, plan, y, ws)
    torch.cuda.synchronize()
    bits = y.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    pad = ybuf[: prob.T, prob.d_out:].float().cpu().numpy()
    assert np.isnan(pad).all(), "fused entry wrote outside the output rows"
    return bits


def _problem(name, T, d_in, d_out, ranks, none_frac, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, len(ranks), T).astype(np.int32)
    ids[rng.random(T) < none_frac] = -1
    base = make_problem(name=name, dtype="bf16", ids=ids, ranks=ranks, alphas=[2.0 * r for r in ranks], d_in=d_in,
                        d_out=d_out, seed=seed, a_std=0.05, b_std=0.05, w0_std=0.05)
    return with_e4m3_base(base, seed=100 + seed, q_std=32.0, w0_std=0.05)


def test_e4m3_every_code_exact():
    """x[t] = e_t (one-hot), no adapters, scale 2^-8: y[t, n] is the value of
    code W0[n, t] times 2^-8, exact in bf16.  W0[n, k] = the (n + k)-th of the
    254 finite codes, so every code appears in every column position."""
    T = d_in = 256
    d_out = 272
    prob = _problem("e4m3_codes", T, d_in, d_out, [8], 1.0, 1)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    n = np.arange(d_out)[:, None]
    k = np.arange(d_in)[None, :]
    codes = finite[(n + k) % finite.size]
    prob.x = f32_to_bf16_bits(np.eye(T, d_in, dtype=np.float32)).reshape(T, d_in)
    prob.W0_e4m3 = codes
    prob.w0_scale = 2.0 ** -8
    say("case e4m3 every finite code")
    bits = run_fused_e4m3(prob)
    y_ref, _ = oracle.lora_forward(prob, fused=True, nthreads=16)
    assert np.array_equal(bits, f32_to_bf16_bits(y_ref.astype(np.float32)))
    vals = oracle.e4m3_decode(codes.T) * 2.0 ** -8  # y[t, n] = value of W0[n, t]
    assert np.array_equal(decode(bits, "bf16"), vals)


def test_e4m3_nan_code_stays_in_its_column():
    """A NaN code in W0[n, k] makes column n NaN for every token (0 * NaN is
    NaN in the oracle too); every other column matches the oracle."""
    prob = _problem("e4m3_nan", 64, 128, 96, [8, 16], 0.2, 2)
    codes = prob.W0_e4m3.copy()
    codes[5, 17] = 0x7F
    codes[40, 100] = 0xFF
    say("case e4m3 NaN codes")
    bits = run_fused_e4m3(prob, codes=codes)
    y = decode(bits, "bf16")
    q = copy.copy(prob)
    q.W0_e4m3 = codes
    y_ref, _ = oracle.lora_forward(q, fused=True, nthreads=16)
    bad = np.isnan(y_ref)
    assert np.array_equal(np.isnan(y), bad)
    assert bad[:, 5].all() and bad[:, 40].all() and bad.sum() == 2 * prob.T
    assert_close(np.where(bad, 0, y), np.where(bad, 0, y_ref), "bf16", "e4m3 NaN codes")


SHAPES = [
    # name, T, d_in, d_out, ranks, none_frac, seed
    ("small_ragged", 37, 64, 40, [8, 16], 0.2, 1),
    ("half_stage_k", 300, 208, 333, [8, 16, 32, 64], 0.1, 2),  # 208 = 6.5 stages of 32
    ("odd_ranks", 260, 144, 200, [5, 12, 1, 33], 0.05, 3),
    ("rank256", 96, 512, 392, [256, 100], 0.0, 4),
    ("many_segments", 520, 256, 584, list(range(1, 41)), 0.05, 5),
    ("all_none", 70, 64, 96, [4], 1.0, 6),
    ("one_token", 1, 128, 192, [16], 0.0, 7),
    ("d_in_16", 48, 16, 200, [8], 0.1, 8),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_e4m3_shapes(shape):
    prob = _problem(*shape)
    name = shape[0]
    say(f"case e4m3 {name} T={prob.T} d_in={prob.d_in} d_out={prob.d_out} scale={prob.w0_scale}")
    bits = run_fused_e4m3(prob)
    y_ref, _ = oracle.lora_forward(prob, fused=True, nthreads=16)
    assert_close(decode(bits, "bf16"), y_ref, "bf16", f"e4m3 {name}")
    say(f"case e4m3 {name} codes=0")
    q = copy.copy(prob)
    q.W0_e4m3 = np.zeros_like(prob.W0_e4m3)
    bits0 = run_fused_e4m3(q)
    y0, _ = oracle.lora_forward(q, fused=True, nthreads=16)
    assert_close(decode(bits0, "bf16"), y0, "bf16", f"e4m3 {name} codes=0")
    if (prob.ids < 0).any():
        assert (decode(bits0, "bf16")[prob.ids < 0] == 0).all()


def test_e4m3_full_size_all_rows():
    """The full-size FP8-base workload: all 1024 x 12288 outputs against the
    oracle, element by element."""
    prob = make_fused_fp8()
    say(f"case e4m3 full-size T={prob.T} d_in={prob.d_in} d_out={prob.d_out}")
    bits = run_fused_e4m3(prob)
    y_ref, _ = oracle.lora_forward(prob, fused=True, nthreads=16)
    assert_close(decode(bits, "bf16"), y_ref, "bf16", "e4m3 full-size")
