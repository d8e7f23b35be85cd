"""Seeded generators: reproducible bytes, the stated structure, exact bf16
rounding, and an unpadded adapter pool."""

import numpy as np
import pytest
import torch

import oracle
from lora_workloads import bf16_bits_to_f32, f32_to_bf16_bits, make_config


def _digest(p):
    parts = [p.ids, p.ranks, p.alphas, p.pool, p.a_off, p.b_off, p.x]
    parts += [a for a in (p.y_in, p.W0) if a is not None]
    return [np.ascontiguousarray(a).tobytes() for a in parts]


@pytest.mark.parametrize("k", [1, 2, 3])
def test_same_seed_same_bytes(k):
    assert _digest(make_config(k)) == _digest(make_config(k))
    assert _digest(make_config(k, seed=100 + k)) != _digest(make_config(k))


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e-39, -2.5e-40],
                                 dtype=np.float32)])
    ours = f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(bf16_bits_to_f32(ours), torch.from_numpy(ours.view(np.int16)).view(
        torch.bfloat16).float().numpy())


def test_config_structure():
    c1 = make_config(1)
    assert c1.ids.tolist() == [0] * 5 + [1] * 3 and c1.dtype == "f32"
    c2 = make_config(2)
    assert c2.T == 64 and c2.n_adapters == 32 and set(c2.ranks.tolist()) == {16}
    assert 20 <= len(c2.distinct_adapters()) <= 32
    c3 = make_config(3)
    lens = c3.meta["segments"]
    assert len(lens) == 16 and sum(lens) == 4096 and min(lens) >= 1
    assert sorted(c3.meta["segment_adapters"]) == list(range(16))
    # contiguous segments
    changes = int(np.count_nonzero(np.diff(c3.ids))) + 1
    assert changes == 16


def test_hetero_pool_is_unpadded():
    """Pool bytes equal sum_i r_i (d_in + d_out) * 2 exactly (no padding)."""
    c4 = make_config(4)
    assert c4.T == 2304 and c4.d_out == 14336
    assert set(c4.ranks.tolist()) <= {8, 16, 32, 64}
    want = sum(oracle.adapter_bytes(int(r), c4.d_in, c4.d_out, 2) for r in c4.ranks)
    assert c4.pool.nbytes == want
    # decode tokens first, then 4 segments of 512 on one adapter each
    assert all(len(set(c4.ids[256 + 512 * s: 256 + 512 * (s + 1)].tolist())) == 1 for s in range(4))


def test_fused_config_structure():
    c5 = make_config(5)
    assert c5.T == 1024 and c5.W0.shape == (12288, 4096) and c5.y_in is None
    lens = c5.meta["requests"]
    assert sum(lens) == 1024 and max(lens) <= 512
    assert c5.n_adapters == 200 and len(c5.meta["resident_ids"]) == 200
    drawn = set(c5.meta["request_adapter"])
    assert drawn <= set(c5.meta["resident_ids"])


def test_prefill_qkv_structure():
    """q, k, v of the prefill batch: the prefill workload's ids for all three,
    one shared x, own adapters and outputs, seeded."""
    from lora_workloads import make_config, make_prefill_qkv

    a, b = make_prefill_qkv(), make_prefill_qkv()
    assert [p.d_out for p in a] == [4096, 1024, 1024]
    assert all(np.array_equal(p.ids, make_config(3).ids) for p in a)
    assert a[1].x is a[0].x and a[2].x is a[0].x
    assert not np.array_equal(a[0].pool[:1000], a[1].pool[:1000])
    for p, q in zip(a, b):
        assert np.array_equal(p.pool, q.pool) and np.array_equal(p.x, q.x)
