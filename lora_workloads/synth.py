"""Seeded synthetic workloads for the multi-LoRA shrink/expand path.

The five named workloads follow the problem as stated on the pages:

* a per-token adapter id (-1 = the token uses no adapter),
* a pool of adapters resident in device memory, each with its own rank r_i and
  scale hyper-parameter alpha_i, stored without padding to a common rank,
* activations x, a base output y (accumulated into) or a base weight W0.

Storage (all row-major, chosen so every contraction operand is contiguous along
its reduction axis):

* x  : [T, d_in]
* A_i: [r_i, d_in]   (the pages' A^T in "x.A.B" notation)
* B_i: [d_out, r_i]  (the pages' B^T)
* W0 : [d_out, d_in]
* y  : [T, d_out]

bf16 arrays are held as uint16 bit patterns (numpy has no bfloat16); they are
produced from float32 draws by round-to-nearest-even.  Random draws happen in a
fixed order: ids/segments, then ranks, then adapters (A_0, B_0, A_1, B_1, ...),
then x, then y_in / W0.  Nothing here computes any part of the LoRA product.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

# Pool offsets are aligned to this many elements (256 B for bf16, 512 B for f32).
POOL_ALIGN_ELEMS = 128

CONFIG_NAMES = {
    1: "tiny_sgmv_f32",
    2: "decode_bgmv_bf16",
    3: "prefill_sgmv_bf16",
    4: "hetero_rank_bf16",
    5: "fused_layer_bf16",
}


def f32_to_bf16_bits(a) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Inputs are finite Gaussian draws, so the NaN/overflow corner of the
    rounding add cannot occur.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exact."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def zipf_probs(n: int, s: float) -> np.ndarray:
    """Truncated Zipf popularity over n ids: P(k) proportional to (k+1)^-s."""
    w = (np.arange(1, n + 1, dtype=np.float64)) ** (-s)
    return w / w.sum()


@dataclass
class LoraProblem:
    """One layer-projection's worth of inputs for the adapter path."""

    name: str
    dtype: str  # "f32" or "bf16"
    T: int
    d_in: int
    d_out: int
    ids: np.ndarray  # int32 [T], -1 = no adapter
    ranks: np.ndarray  # int32 [N]
    alphas: np.ndarray  # float32 [N]
    pool: np.ndarray  # flat storage (uint16 bf16 bits or float32)
    a_off: np.ndarray  # int64 [N], element offset of A_i in pool
    b_off: np.ndarray  # int64 [N], element offset of B_i in pool
    x: np.ndarray  # [T, d_in]
    y_in: Optional[np.ndarray]  # [T, d_out] base output to accumulate into (None = zeros)
    W0: Optional[np.ndarray]  # [d_out, d_in] base weight for the fused entry
    meta: dict = field(default_factory=dict)
    # FP8 base: [d_out, d_in] uint8 E4M3 codes standing for w0_scale * code
    # (W0 is then None)
    W0_e4m3: Optional[np.ndarray] = None
    w0_scale: float = 1.0

    @property
    def n_adapters(self) -> int:
        return int(self.ranks.shape[0])

    @property
    def esize(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def max_rank(self) -> int:
        return int(self.ranks.max()) if self.ranks.size else 0

    def A(self, i: int) -> np.ndarray:
        r = int(self.ranks[i])
        o = int(self.a_off[i])
        return self.pool[o : o + r * self.d_in].reshape(r, self.d_in)

    def B(self, i: int) -> np.ndarray:
        r = int(self.ranks[i])
        o = int(self.b_off[i])
        return self.pool[o : o + self.d_out * r].reshape(self.d_out, r)

    def to_f32(self, arr: np.ndarray) -> np.ndarray:
        """Decode a stored array to float32 (exact for both dtypes)."""
        if self.dtype == "bf16":
            return bf16_bits_to_f32(arr).reshape(arr.shape)
        return np.asarray(arr, dtype=np.float32)

    def y_base(self) -> np.ndarray:
        """The stored base output (zeros when none was drawn)."""
        if self.y_in is not None:
            return self.y_in
        dt = np.uint16 if self.dtype == "bf16" else np.float32
        return np.zeros((self.T, self.d_out), dtype=dt)

    def distinct_adapters(self) -> np.ndarray:
        ids = self.ids[self.ids >= 0]
        return np.unique(ids)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(a).reshape(a.shape)
    return np.ascontiguousarray(a, dtype=np.float32)


def _pool_layout(ranks: np.ndarray, d_in: int, d_out: int):
    """Element offsets of A_i and B_i in an unpadded pool (each start aligned)."""
    def up(v):
        return (v + POOL_ALIGN_ELEMS - 1) // POOL_ALIGN_ELEMS * POOL_ALIGN_ELEMS

    a_off = np.zeros(len(ranks), dtype=np.int64)
    b_off = np.zeros(len(ranks), dtype=np.int64)
    cur = 0
    for i, r in enumerate(ranks):
        r = int(r)
        a_off[i] = cur
        cur = up(cur + r * d_in)
        b_off[i] = cur
        cur = up(cur + d_out * r)
    return a_off, b_off, cur


def _fill_pool(rng, ranks, d_in, d_out, a_std, b_std, dtype, zero_adapters=()):
    a_off, b_off, total = _pool_layout(ranks, d_in, d_out)
    dt = np.uint16 if dtype == "bf16" else np.float32
    pool = np.zeros(total, dtype=dt)
    for i, r in enumerate(ranks):
        r = int(r)
        a = rng.standard_normal(r * d_in, dtype=np.float32) * np.float32(a_std)
        b = rng.standard_normal(d_out * r, dtype=np.float32) * np.float32(b_std)
        if i in zero_adapters:
            a[:] = 0
            b[:] = 0
        pool[a_off[i] : a_off[i] + r * d_in] = _store(a, dtype)
        pool[b_off[i] : b_off[i] + d_out * r] = _store(b, dtype)
    return pool, a_off, b_off


def make_problem(
    *,
    name: str,
    dtype: str,
    ids: Sequence[int],
    ranks: Sequence[int],
    alphas: Sequence[float],
    d_in: int,
    d_out: int,
    seed: int,
    x_std: float = 1.0,
    a_std: float = 0.02,
    b_std: float = 0.02,
    y_mode: str = "normal",  # "normal" | "zero"
    w0_std: Optional[float] = None,
    rng: Optional[np.random.Generator] = None,
    meta: Optional[dict] = None,
) -> LoraProblem:
    """Generic seeded problem: structure is given, values are drawn here.

    Draw order after the structure: adapters, x, then y_in (if "normal"), then
    W0 (if w0_std is given).
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    ids = np.asarray(ids, dtype=np.int32)
    ranks = np.asarray(ranks, dtype=np.int32)
    alphas = np.asarray(alphas, dtype=np.float32)
    T = int(ids.shape[0])
    pool, a_off, b_off = _fill_pool(rng, ranks, d_in, d_out, a_std, b_std, dtype)
    x = _store(rng.standard_normal((T, d_in), dtype=np.float32) * np.float32(x_std), dtype)
    y_in = None
    if y_mode == "normal":
        y_in = _store(rng.standard_normal((T, d_out), dtype=np.float32), dtype)
    elif y_mode != "zero":
        raise ValueError(y_mode)
    W0 = None
    if w0_std is not None:
        W0 = _store(rng.standard_normal((d_out, d_in), dtype=np.float32) * np.float32(w0_std), dtype)
    return LoraProblem(
        name=name, dtype=dtype, T=T, d_in=d_in, d_out=d_out, ids=ids, ranks=ranks,
        alphas=alphas, pool=pool, a_off=a_off, b_off=b_off, x=x, y_in=y_in, W0=W0,
        meta=dict(meta or {}),
    )


def e4m3_codes(a) -> np.ndarray:
    """float32 values -> uint8 E4M3 codes by torch's float8_e4m3fn cast (round to
    nearest even); values are first clipped to the format's largest finite
    magnitude, 448, so that none becomes NaN."""
    import torch

    a = np.clip(np.ascontiguousarray(a, dtype=np.float32), -448.0, 448.0)
    return torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def with_e4m3_base(prob: LoraProblem, seed: int, q_std: float = 32.0, w0_std: float = 0.02,
                   name: Optional[str] = None) -> LoraProblem:
    """The same problem with its base weight replaced by an FP8 one: codes of
    Gaussian draws with standard deviation q_std (so that the codes use the
    format's range) and one fp32 scale w0_std / q_std, so that the weight the
    codes stand for has standard deviation w0_std.  Draws from its own seed."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((prob.d_out, prob.d_in), dtype=np.float32) * np.float32(q_std)
    import copy

    out = copy.copy(prob)
    out.W0 = None
    out.W0_e4m3 = e4m3_codes(q)
    out.w0_scale = float(np.float32(w0_std / q_std))
    out.meta = dict(prob.meta, fused=True, w0_format="e4m3")
    if name is not None:
        out.name = name
    return out


FUSED_FP8_NAME = "fused_layer_fp8w_bf16"


def make_fused_fp8(seed: int = 5) -> LoraProblem:
    """The fused-layer workload (1024 tokens, Zipf requests over 200 resident
    rank-16 slots, W0 [12288, 4096], y overwritten) with an FP8 E4M3 base of
    one fp32 scale, weight std 0.02 as in the bf16 form; adapters, x and the
    plan are those of the bf16 workload with the same seed."""
    return with_e4m3_base(make_config(5, seed), seed=1000 + seed, name=FUSED_FP8_NAME)


def dirichlet_lengths(rng, total: int, k: int) -> np.ndarray:
    """k segment lengths summing to total, each >= 1, from a Dirichlet(1) split.

    L_k = 1 + floor(p_k * (total - k)); the remainder goes one token each to the
    largest fractional parts (ties to the lower index).
    """
    p = rng.dirichlet(np.ones(k))
    share = p * (total - k)
    base = np.floor(share).astype(np.int64)
    frac = share - base
    lens = 1 + base
    rem = total - int(lens.sum())
    order = sorted(range(k), key=lambda i: (-frac[i], i))
    for i in order[:rem]:
        lens[i] += 1
    assert int(lens.sum()) == total and lens.min() >= 1
    return lens


def geometric_requests(rng, total: int, p: float, cap: int) -> np.ndarray:
    """Request lengths min(Geometric(p), cap) until the sum reaches total; the
    last one is cut so that the lengths sum to exactly total."""
    lens = []
    s = 0
    while s < total:
        L = int(min(rng.geometric(p), cap))
        L = min(L, total - s)
        lens.append(L)
        s += L
    return np.asarray(lens, dtype=np.int64)


def make_config(k: int, seed: Optional[int] = None) -> LoraProblem:
    """The five named workloads (k = 1..5).  Default seed = k."""
    if seed is None:
        seed = k
    rng = np.random.default_rng(seed)
    name = CONFIG_NAMES[k]
    if k == 1:
        # 8 tokens in two segments [5, 3] on adapters [0, 1]; d = 256; r = 8; alpha = 16.
        ids = [0] * 5 + [1] * 3
        d = 256
        return make_problem(
            name=name, dtype="f32", ids=ids, ranks=[8, 8], alphas=[16.0, 16.0], d_in=d, d_out=d,
            seed=seed, rng=rng, x_std=1.0 / 16.0, a_std=1.0 / 16.0, b_std=1.0 / np.sqrt(8.0),
            y_mode="zero", w0_std=1.0 / 16.0, meta={"segments": [5, 3]},
        )
    if k == 2:
        # 64 one-token rows, adapter per token uniform over a pool of 32; d = 4096; r = 16.
        ids = rng.integers(0, 32, 64).astype(np.int32)
        return make_problem(
            name=name, dtype="bf16", ids=ids, ranks=[16] * 32, alphas=[32.0] * 32,
            d_in=4096, d_out=4096, seed=seed, rng=rng,
        )
    if k == 3:
        # 4096 tokens in 16 contiguous Dirichlet(1) segments, segment k -> adapter perm16[k].
        lens = dirichlet_lengths(rng, 4096, 16)
        perm16 = rng.permutation(16)
        ids = np.repeat(perm16.astype(np.int32), lens)
        return make_problem(
            name=name, dtype="bf16", ids=ids, ranks=[16] * 16, alphas=[32.0] * 16,
            d_in=4096, d_out=4096, seed=seed, rng=rng,
            meta={"segments": lens.tolist(), "segment_adapters": perm16.tolist()},
        )
    if k == 4:
        # 256 decode tokens + 4 prefill segments of 512; Zipf(1.1) popularity over 128
        # adapters; ranks uniform over {8,16,32,64}, unpadded; d_in 4096, d_out 14336.
        P = zipf_probs(128, 1.1)
        dec = rng.choice(128, size=256, p=P).astype(np.int32)
        pre = rng.choice(128, size=4, p=P).astype(np.int32)
        ids = np.concatenate([dec, np.repeat(pre, 512)]).astype(np.int32)
        ranks = rng.choice(np.array([8, 16, 32, 64], dtype=np.int32), size=128)
        return make_problem(
            name=name, dtype="bf16", ids=ids, ranks=ranks, alphas=[32.0] * 128,
            d_in=4096, d_out=14336, seed=seed, rng=rng,
            meta={"decode_tokens": 256, "prefill_segments": pre.tolist()},
        )
    if k == 5:
        # 1024 tokens in requests of geometric(0.05) length (cap 512); request adapter
        # Zipf(1.1) over 1000; 200 resident rank-16 slots; W0 [12288, 4096]; y overwritten.
        lens = geometric_requests(rng, 1024, 0.05, 512)
        P = zipf_probs(1000, 1.1)
        req_adapter = rng.choice(1000, size=len(lens), p=P)
        drawn = sorted(set(int(a) for a in req_adapter))
        resident = list(drawn)
        for a in range(1000):  # fill the remaining slots with the most popular ids
            if len(resident) >= 200:
                break
            if a not in drawn:
                resident.append(a)
        resident = sorted(resident)
        slot_of = {a: s for s, a in enumerate(resident)}
        ids = np.repeat(np.array([slot_of[int(a)] for a in req_adapter], dtype=np.int32), lens)
        return make_problem(
            name=name, dtype="bf16", ids=ids, ranks=[16] * 200, alphas=[32.0] * 200,
            d_in=4096, d_out=12288, seed=seed, rng=rng, y_mode="zero", w0_std=0.02,
            meta={"requests": lens.tolist(), "request_adapter": [int(a) for a in req_adapter],
                  "resident_ids": resident, "fused": True},
        )
    raise ValueError(f"unknown config {k}")


QKV_NAME = "decode_qkv_grouped_bf16"


def make_decode_qkv(seed: int = 2, d_outs: Sequence[int] = (4096, 1024, 1024)) -> list:
    """The q, k and v projections of one decode batch, for the grouped call: the
    decode workload's 64 tokens, ids (uniform over a pool of 32 adapters of rank
    16, alpha 32) and value distributions, d_in 4096, d_out 4096 / 1024 / 1024
    (grouped-query attention with a quarter of the heads for k and v).  One id
    per token for all three projections; x is shared (the same array object);
    every projection has its own adapters (A, B) and base output."""
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, 32, 64).astype(np.int32)
    probs = []
    for p, d_out in enumerate(d_outs):
        prob = make_problem(name=f"{QKV_NAME}/{'qkv'[p] if p < 3 else p}", dtype="bf16", ids=ids, ranks=[16] * 32,
                            alphas=[32.0] * 32, d_in=4096, d_out=d_out, seed=seed, rng=rng)
        if p > 0:
            prob.x = probs[0].x
        probs.append(prob)
    return probs


PREFILL_QKV_NAME = "prefill_qkv_grouped_bf16"


def make_prefill_qkv(seed: int = 3, d_outs: Sequence[int] = (4096, 1024, 1024)) -> list:
    """The q, k and v projections of one prefill batch, for the grouped SGMV
    call: the prefill workload's 4096 tokens in 16 Dirichlet(1) segments over
    a pool of 16 rank-16 adapters (alpha 32), d_in 4096, d_out 4096 / 1024 /
    1024.  One id per token for all three projections; x is shared (the same
    array object); every projection has its own adapters and base output."""
    ids = make_config(3, seed=seed).ids
    rng = np.random.default_rng(seed + 7)
    probs = []
    for p, d_out in enumerate(d_outs):
        prob = make_problem(name=f"{PREFILL_QKV_NAME}/{'qkv'[p] if p < 3 else p}", dtype="bf16", ids=ids,
                            ranks=[16] * 16, alphas=[32.0] * 16, d_in=4096, d_out=d_out, seed=seed, rng=rng)
        if p > 0:
            prob.x = probs[0].x
        probs.append(prob)
    return probs


CACHE_NAME = "decode_cache_bf16"


def make_decode_registry(seed: int = 2, n_adapters: int = 256, n_batches: int = 64):
    """Decode batches over an adapter registry larger than HBM is given for it:
    n_adapters adapters of rank 16 (alpha 32, d 4096 -> 4096, values as in the
    decode workload), and n_batches id lists of 64 tokens drawn from a
    Zipf(1.1) popularity over the registry (the pages' benchmark protocol).
    Returns (problem holding every adapter and batch 0's tokens, [ids per batch])."""
    rng = np.random.default_rng(seed)
    P = zipf_probs(n_adapters, 1.1)
    batches = [rng.choice(n_adapters, size=64, p=P).astype(np.int32) for _ in range(n_batches)]
    prob = make_problem(name=CACHE_NAME, dtype="bf16", ids=batches[0], ranks=[16] * n_adapters,
                        alphas=[32.0] * n_adapters, d_in=4096, d_out=4096, seed=seed, rng=rng)
    return prob, batches


def make_integer_problem(
    *, seed: int, dtype: str, T: int, d_in: int, d_out: int, n_adapters: int,
    ranks: Optional[Sequence[int]] = None, with_w0: bool = False, none_frac: float = 0.0,
) -> LoraProblem:
    """Tiny problem whose entries are in {-1, 0, 1} and whose scale is 1 (alpha = r).

    Every partial sum of the product is then a small integer, exactly
    representable in fp32 and bf16, so any correct summation order gives the
    same bits.  y_in entries are drawn from {-1, 1} (never -0) and W0 from
    {-1, 0, 1}.
    """
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, n_adapters, T).astype(np.int32)
    if none_frac > 0:
        ids[rng.random(T) < none_frac] = -1
    if ranks is None:
        ranks = rng.integers(1, 5, n_adapters)
    ranks = np.asarray(ranks, dtype=np.int32)
    alphas = ranks.astype(np.float32)
    a_off, b_off, total = _pool_layout(ranks, d_in, d_out)
    pool = np.zeros(total, dtype=np.float32)
    for i, r in enumerate(ranks):
        r = int(r)
        pool[a_off[i] : a_off[i] + r * d_in] = rng.integers(-1, 2, r * d_in)
        pool[b_off[i] : b_off[i] + d_out * r] = rng.integers(-1, 2, d_out * r)
    x = rng.integers(-1, 2, (T, d_in)).astype(np.float32)
    y_in = rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=(T, d_out))
    W0 = rng.integers(-1, 2, (d_out, d_in)).astype(np.float32) if with_w0 else None
    return LoraProblem(
        name="integer", dtype=dtype, T=T, d_in=d_in, d_out=d_out, ids=ids, ranks=ranks,
        alphas=alphas, pool=_store(pool, dtype), a_off=a_off, b_off=b_off, x=_store(x, dtype),
        y_in=_store(y_in, dtype), W0=None if W0 is None else _store(W0, dtype),
    )
