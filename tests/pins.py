"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each ``pin_*`` function raises AssertionError when the oracle (built with the
given planted-mistake id; 0 = the real one) disagrees with what the pages or
the mathematics fix.  They are run against the real oracle in
test_oracle_pins.py and against every planted mistake in
test_oracle_mutants.py, which checks that each mistake is caught by at least
one pin.

Independent references used here: the pages' printed numbers
(tests/golden/adapter_sizes.json), numpy matrix products (a library routine,
not the oracle's loops), exact integer arithmetic in pure Python, Python's
stable ``sorted``, and special cases (zero adapter, scale doubling, padding).
For the E4M3 decode: the values the OCP 8-bit floating point specification
names (tests/golden/e4m3_values.json), torch's float8_e4m3fn conversion (a
library routine), an exact pure-Python decode with fractions, and the
format's structure (order, spacing, symmetry).
"""

from __future__ import annotations

import json
import os

import numpy as np

import oracle
from lora_workloads import make_config, make_integer_problem, make_problem

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f64(prob, arr):
    return prob.to_f32(arr).astype(np.float64)


def _correction_numpy(prob, ids=None):
    """s * (x A_a^T) B_a^T per token group, with numpy matmuls (fp64)."""
    ids = prob.ids if ids is None else ids
    x = _f64(prob, prob.x)
    out = np.zeros((prob.T, prob.d_out))
    for a in np.unique(ids[ids >= 0]):
        rows = np.nonzero(ids == a)[0]
        A = _f64(prob, prob.A(a))
        B = _f64(prob, prob.B(a))
        s = float(prob.alphas[a]) / float(prob.ranks[a])
        out[rows] = s * ((x[rows] @ A.T) @ B.T)
    return out


# ---------------------------------------------------------------- size formula
def pin_adapter_sizes(mutant=0):
    """The pages' printed adapter sizes, rebuilt from r (d_in + d_out)."""
    with open(os.path.join(GOLDEN, "adapter_sizes.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        per_layer = sum(oracle.adapter_bytes(c["r"], di, do, c["bytes_per_param"], mutant=mutant)
                        for di, do in c["mats"])
        total = per_layer * c["layers"] * c.get("copies", 1)
        unit = c["unit"]
        got = {"B": total, "params": total, "MiB": total / 2**20, "MB": total / 1e6,
               "GB": total / 1e9, "Mparams": total / 1e6}[unit]
        tol = c["rel_tol"] * abs(c["value"])
        assert abs(got - c["value"]) <= tol, (c["source"], got, c["value"])


# ---------------------------------------------------------------- merge identity
def pin_merge_identity(mutant=0):
    """x (W0 + s B A) == x W0 + s (x A) B for one adapter on every token.

    The right side is the oracle's fused run (its own loops for x W0, its own
    shrink/expand); the left side merges the weights and multiplies with numpy.
    """
    for prob in (make_config(1), make_problem(name="merge", dtype="bf16", ids=[0] * 7, ranks=[5],
                                              alphas=[3.0], d_in=40, d_out=24, seed=11, a_std=0.3,
                                              b_std=0.3, w0_std=0.2, y_mode="zero")):
        ids = np.zeros(prob.T, dtype=np.int32)  # every token on adapter 0
        y, _ = oracle.lora_forward(prob, ids=ids, fused=True, mutant=mutant)
        s = float(prob.alphas[0]) / float(prob.ranks[0])
        W = _f64(prob, prob.W0) + s * (_f64(prob, prob.B(0)) @ _f64(prob, prob.A(0)))
        ref = _f64(prob, prob.x) @ W.T
        err = np.max(np.abs(y - ref) / (np.abs(ref) + 1e-3))
        assert err < 1e-11, err


# ---------------------------------------------------------------- homogeneous / mixed
def pin_homogeneous_and_mixed(mutant=0):
    """(i) all tokens on one adapter: correction == numpy s (X A^T) B^T.
    (ii) mixed adapters (heterogeneous ranks, some tokens with none): each
    token's correction equals its own adapter's numpy product."""
    p1 = make_config(1)
    for a in range(p1.n_adapters):
        ids = np.full(p1.T, a, dtype=np.int32)
        y, _ = oracle.lora_forward(p1, ids=ids, mutant=mutant)
        ref = _correction_numpy(p1, ids)
        assert np.max(np.abs(y - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref))), a
    rng = np.random.default_rng(5)
    ids = rng.integers(-1, 6, 29).astype(np.int32)
    prob = make_problem(name="mixed", dtype="bf16", ids=ids, ranks=[1, 3, 8, 16, 5, 2],
                        alphas=[2.0, 6.0, 16.0, 8.0, 5.0, 7.0], d_in=72, d_out=40, seed=6,
                        a_std=0.2, b_std=0.2)
    y, _ = oracle.lora_forward(prob, mutant=mutant)
    ref = _correction_numpy(prob) + _f64(prob, prob.y_in)
    assert np.max(np.abs(y - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref)))


# ---------------------------------------------------------------- exact brute force
def pin_integer_bruteforce(mutant=0):
    """Entries in {-1,0,1}, alpha = r (scale 1): pure-Python integer arithmetic
    gives the exact result, which the fp64 oracle must reproduce exactly."""
    for seed in (1, 2, 3):
        for with_w0 in (False, True):
            prob = make_integer_problem(seed=seed, dtype="f32", T=7, d_in=9, d_out=6,
                                        n_adapters=3, with_w0=with_w0, none_frac=0.2)
            y, v = oracle.lora_forward(prob, want_v=True, fused=with_w0, mutant=mutant)
            X = [[int(u) for u in row] for row in prob.x]
            for t in range(prob.T):
                a = int(prob.ids[t])
                for n in range(prob.d_out):
                    if with_w0:
                        base = sum(X[t][k] * int(prob.W0[n][k]) for k in range(prob.d_in))
                    else:
                        base = int(prob.y_in[t][n])
                    corr = 0
                    if a >= 0:
                        A = prob.A(a)
                        B = prob.B(a)
                        vv = [sum(X[t][k] * int(A[j][k]) for k in range(prob.d_in))
                              for j in range(int(prob.ranks[a]))]
                        corr = sum(vv[j] * int(B[n][j]) for j in range(len(vv)))
                        if n == 0:
                            assert list(v[t, : len(vv)]) == vv, (t, v[t], vv)
                    assert y[t, n] == base + corr, (seed, t, n, y[t, n], base + corr)


# ---------------------------------------------------------------- special cases
def pin_zero_adapter_and_none(mutant=0):
    """B = 0 or A = 0 leaves y_in untouched; so does id -1."""
    rng = np.random.default_rng(9)
    ids = rng.integers(-1, 3, 21).astype(np.int32)
    prob = make_problem(name="zero", dtype="bf16", ids=ids, ranks=[4, 7, 2], alphas=[1.0, 2.0, 3.0],
                        d_in=33, d_out=17, seed=10)
    y_in = _f64(prob, prob.y_in)
    for which in ("A", "B"):
        pool = prob.pool.copy()
        for a in range(prob.n_adapters):
            if which == "A":
                o, n = prob.a_off[a], prob.ranks[a] * prob.d_in
            else:
                o, n = prob.b_off[a], prob.ranks[a] * prob.d_out
            pool[o : o + n] = 0
        y, _ = oracle.lora_forward(prob, pool=pool, mutant=mutant)
        assert np.array_equal(y, y_in), which
    y, _ = oracle.lora_forward(prob, ids=np.full(prob.T, -1, dtype=np.int32), mutant=mutant)
    assert np.array_equal(y, y_in)


def pin_scale_linearity(mutant=0):
    """With a zero base, doubling every alpha doubles the output exactly."""
    p = make_config(1)
    y1, _ = oracle.lora_forward(p, mutant=mutant)
    y2, _ = oracle.lora_forward(p, alphas=p.alphas * 2, mutant=mutant)
    assert np.array_equal(y2, 2 * y1)
    assert np.max(np.abs(y1)) > 0


def pin_padding_invariance(mutant=0):
    """Zero-padding A_i, B_i from r_i to r' (alpha scaled by r'/r_i so that
    alpha/r is unchanged) gives the same output: ranks need no padding."""
    rng = np.random.default_rng(12)
    ids = rng.integers(0, 3, 11).astype(np.int32)
    ranks = [2, 4, 8]
    prob = make_problem(name="pad", dtype="f32", ids=ids, ranks=ranks, alphas=[4.0, 8.0, 16.0],
                        d_in=24, d_out=20, seed=13, a_std=0.5, b_std=0.5)
    y, _ = oracle.lora_forward(prob, mutant=mutant)
    rp = 16
    padded = make_problem(name="pad16", dtype="f32", ids=ids, ranks=[rp] * 3,
                          alphas=[4.0 * rp / 2, 8.0 * rp / 4, 16.0 * rp / 8], d_in=24, d_out=20,
                          seed=0, a_std=0.0, b_std=0.0)
    padded.x[:] = prob.x
    padded.y_in[:] = prob.y_in
    for a, r in enumerate(ranks):
        padded.A(a)[:r, :] = prob.A(a)
        padded.B(a)[:, :r] = prob.B(a)
    yp, _ = oracle.lora_forward(padded, mutant=mutant)
    assert np.allclose(yp, y, rtol=1e-13, atol=1e-13)


def pin_nan_locality(mutant=0):
    """A NaN in x[t] makes only row t non-finite."""
    prob = make_config(1)
    prob.x = prob.x.copy()
    prob.x[3, 17] = np.nan
    y, _ = oracle.lora_forward(prob, mutant=mutant)
    bad = ~np.isfinite(y).all(axis=1)
    assert bad.tolist() == [t == 3 for t in range(prob.T)]


# ---------------------------------------------------------------- E4M3 decode
def _e4m3_exact(code: int):
    """Exact value of an E4M3 code as a Fraction (None for NaN), from the
    format's definition: sign, 4-bit exponent field (bias 7), 3-bit mantissa;
    exponent field 0 is subnormal; S.1111.111 is NaN."""
    from fractions import Fraction

    sign = -1 if code & 0x80 else 1
    e, m = (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return None
    if e == 0:
        mag = Fraction(m, 8) * Fraction(1, 2**6)
    else:
        mag = Fraction(8 + m, 8) * (Fraction(2) ** (e - 7))
    return sign * mag


def pin_e4m3_decode(mutant=0):
    """All 256 codes: the values the specification names, torch's
    float8_e4m3fn decode, an exact decode with fractions, and the format's
    structure."""
    import math

    import torch

    got = oracle.e4m3_decode(np.arange(256, dtype=np.uint8), mutant=mutant)
    with open(os.path.join(GOLDEN, "e4m3_values.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        v = got[c["code"]]
        if c["value"] is None:
            assert math.isnan(v), c
        else:
            want = math.ldexp(c["value"][0], c["value"][1])
            assert v == want and math.copysign(1.0, v) == math.copysign(1.0, want), (c, v)
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(lib))
    fin = ~np.isnan(lib)
    assert np.array_equal(got[fin], lib[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(lib[fin]))
    for code in range(256):
        ex = _e4m3_exact(code)
        assert (ex is None) == math.isnan(got[code]), code
        if ex is not None:
            assert got[code] == float(ex), (code, got[code], ex)
    pos = got[:127]  # +0 .. 448
    assert np.all(np.diff(pos) > 0)  # codes 0x00 .. 0x7E increase strictly
    assert np.array_equal(got[128:255], -pos)  # sign bit mirrors
    for e in range(1, 16):  # normals: 8 values per binade, equally spaced
        vals = got[8 * e : 8 * e + (7 if e == 15 else 8)]
        assert np.all(np.diff(vals) == vals[0] / 8)
    assert np.all(np.diff(got[0:9]) == got[1])  # subnormals continue the spacing of the first binade
    assert int(np.isnan(got).sum()) == 2


def pin_e4m3_base(mutant=0):
    """The layer over an FP8 base: with a power-of-two scale every weight
    w0_scale * q is exact in bf16, and the output equals the oracle's bf16-base
    output for those weights (converted by torch's float8 decode, not the
    oracle's); a scale of three times that gives three times the base product
    (no adapters)."""
    import copy

    import torch

    from lora_workloads import bf16_bits_to_f32, f32_to_bf16_bits, with_e4m3_base

    rng = np.random.default_rng(41)
    ids = rng.integers(-1, 3, 13).astype(np.int32)
    prob = make_problem(name="fp8base", dtype="bf16", ids=ids, ranks=[4, 8, 2], alphas=[8.0, 4.0, 6.0],
                        d_in=48, d_out=20, seed=42, a_std=0.2, b_std=0.2, y_mode="zero", w0_std=0.1)
    q = with_e4m3_base(prob, seed=43, q_std=40.0)
    q.w0_scale = 2.0 ** -8
    y8, _ = oracle.lora_forward(q, fused=True, mutant=mutant)
    wq = torch.from_numpy(q.W0_e4m3).view(torch.float8_e4m3fn).to(torch.float32).numpy() * np.float32(2.0 ** -8)
    b = copy.copy(prob)
    b.W0 = f32_to_bf16_bits(wq).reshape(wq.shape)
    assert np.array_equal(bf16_bits_to_f32(b.W0).reshape(wq.shape), wq)  # exact in bf16
    yb, _ = oracle.lora_forward(b, fused=True, mutant=mutant)
    assert np.max(np.abs(y8 - yb)) <= 1e-12 * max(1.0, np.max(np.abs(yb)))
    none = np.full(q.T, -1, dtype=np.int32)
    y1, _ = oracle.lora_forward(q, ids=none, fused=True, mutant=mutant)
    q3 = copy.copy(q)
    q3.w0_scale = 3 * 2.0 ** -8
    y3, _ = oracle.lora_forward(q3, ids=none, fused=True, mutant=mutant)
    assert np.max(np.abs(y3 - 3 * y1)) <= 1e-12 * np.max(np.abs(y3))
    assert np.max(np.abs(y1)) > 0


# ---------------------------------------------------------------- segments
def pin_segments(mutant=0):
    """Segments equal Python's stable sort of token indices by id (ids < 0
    dropped), split at id changes."""
    rng = np.random.default_rng(21)
    for T, N in ((0, 3), (1, 1), (17, 4), (200, 9), (64, 32)):
        ids = rng.integers(-1, N, T).astype(np.int32)
        perm, indptr, adapter = oracle.segments(ids, N, mutant=mutant)
        order = sorted([t for t in range(T) if ids[t] >= 0], key=lambda t: ids[t])
        assert perm.tolist() == order
        keys = [int(ids[t]) for t in order]
        bounds = [0] + [p for p in range(1, len(keys)) if keys[p] != keys[p - 1]] + [len(keys)]
        if not keys:
            bounds = [0]
        assert indptr.tolist() == bounds
        assert adapter.tolist() == [keys[b] for b in bounds[:-1]]


ALL_PINS = [
    pin_adapter_sizes,
    pin_merge_identity,
    pin_homogeneous_and_mixed,
    pin_integer_bruteforce,
    pin_zero_adapter_and_none,
    pin_scale_linearity,
    pin_padding_invariance,
    pin_nan_locality,
    pin_segments,
    pin_e4m3_decode,
    pin_e4m3_base,
]

# Planted mistakes compiled into oracle.c with -DORACLE_MUTANT=k.
MUTANTS = {
    1: "A read transposed",
    2: "scale dropped",
    3: "scale inverted",
    4: "base overwritten instead of accumulated into",
    5: "B read transposed",
    6: "last term of the shrink sum dropped",
    7: "neighbouring token's adapter used",
    8: "order within a segment reversed",
    9: "size formula parenthesis dropped",
    10: "correction sign flipped",
    11: "E4M3 exponent bias 8",
    12: "E4M3 subnormals given the implicit one",
    13: "FP8 base scale dropped",
    14: "E4M3 NaN pattern decoded as a number",
}


def failing_pins(mutant):
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    return failed
