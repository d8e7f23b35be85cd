"""Host-side logic of the adapter residency cache (lora_cache_*), run in its
placement-only mode (LORA_CACHE_DRY: no GPU call, no copy): unpadded extents,
least-recently-used eviction, pinning, merging of freed space, capacity and
fragmentation errors, argument checks."""

import ctypes

import numpy as np
import pytest

from segmented_gather_gemm_lora_amd import binding as B

D_IN, D_OUT = 4096, 1024
BASE = 0x7F0000000000


def extent(r, es=2):
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    return up(r * D_IN * es) + up(D_OUT * r * es)


def cache_for(units_of_rank16, n=16, ranks=None, dtype="bf16"):
    tab = B.load().lora_cache_table_bytes(n)
    c = B.AdapterCache.dry_run(tab + units_of_rank16 * extent(16), n, dtype, D_IN, D_OUT)
    host = np.zeros(8, dtype=np.uint16)  # never read in dry mode
    for a in range(n):
        c.register(a, host, host, (ranks or {}).get(a, 16), 32.0)
    return c, tab


def resident(c):
    A, _, r, _ = c.host_tables()
    return {a for a in range(c.n_adapters) if A[a] != 0}


def test_table_bytes_and_extents():
    lib = B.load()
    assert lib.lora_cache_table_bytes(10) == 256  # 240 B of tables, 256-aligned
    assert lib.lora_cache_table_bytes(100) == 2560
    c, tab = cache_for(8, ranks={0: 8, 1: 16, 2: 64})
    c.prepare([0, 1, 2, -1, 1])
    st = c.stats()
    assert st["misses"] == 3 and st["hits"] == 0 and st["resident"] == 3
    assert st["resident_bytes"] == extent(8) + extent(16) + extent(64)
    assert st["bytes_copied"] == 2 * (8 + 16 + 64) * (D_IN + D_OUT)  # no padding to the largest rank
    A, Bt, r, al = c.host_tables()
    # first fit from the start of the data region; B follows A inside the extent
    assert A[0] == BASE + tab and Bt[0] == A[0] + 8 * D_IN * 2
    assert A[1] == BASE + tab + extent(8)
    assert list(r[:4]) == [8, 16, 64, 0] and al[0] == 32.0 and A[3] == 0
    v = c.view()
    assert v.pool_A_dev == BASE and v.rank_dev == BASE + 16 * 16 and v.max_rank == 64


def test_lru_eviction_order():
    c, _ = cache_for(3)
    c.prepare([0, 1, 2])            # batch 0
    c.prepare([1])                  # batch 1: hit
    c.prepare([3])                  # batch 2: evicts 0 (least recently used)
    assert resident(c) == {1, 2, 3}
    c.prepare([0, 3])               # batch 3: evicts 2 (last used in batch 0)
    assert resident(c) == {0, 1, 3}
    st = c.stats()
    assert (st["hits"], st["misses"], st["evictions"], st["batches"]) == (2, 5, 2, 4)


def test_adapters_of_the_batch_are_never_evicted():
    c, _ = cache_for(3)
    c.prepare([0, 1, 2])
    c.prepare([2, 1, 4])            # 0 is the only candidate
    assert resident(c) == {1, 2, 4}


def test_pinned_adapters_stay():
    c, _ = cache_for(3)
    c.pin(0)
    c.prepare([0, 1, 2])
    for a in (3, 4, 5, 6):
        c.prepare([a])
        assert 0 in resident(c)
    c.pin(0, False)
    c.prepare([7])
    c.prepare([8])
    assert 0 not in resident(c)


def test_freed_space_is_merged():
    """Two evicted neighbours hold one adapter of twice the rank."""
    c, tab = cache_for(4, ranks={9: 32})
    c.prepare([0, 1, 2, 3])
    A0 = c.host_tables()[0][0]
    c.prepare([2, 3])
    c.prepare([9])                  # needs two rank-16 extents: evicts 0 then 1, merged
    assert resident(c) == {2, 3, 9}
    assert c.host_tables()[0][9] == A0
    assert c.stats()["evictions"] == 2


def test_batch_larger_than_cache():
    c, _ = cache_for(2)
    with pytest.raises(B.LoraError) as e:
        c.prepare([0, 1, 2])
    assert e.value.status == -6
    c.pin(0)
    c.prepare([0])
    with pytest.raises(B.LoraError):
        c.prepare([1, 2])           # 0 is pinned: one extent left
    c.prepare([1])


def test_fragmentation_error():
    """Pinned adapters split the free space: a rank-32 adapter has room in
    bytes but not in one piece."""
    c, _ = cache_for(4, ranks={9: 32})
    c.pin(0)
    c.pin(2)
    c.prepare([0, 1, 2, 3])
    with pytest.raises(B.LoraError) as e:
        c.prepare([9])
    assert e.value.status == -6 and "fragmented" in B.load().lora_last_error().decode()


def test_failed_prepare_leaves_cache_unchanged():
    """A batch that cannot be placed changes nothing: adapters placed before
    the failure are not left resident without their copy, victims are not
    evicted, and the next batch that needs them counts a miss and copies."""
    c, _ = cache_for(6, ranks={9: 32})
    for a in (0, 2, 4):
        c.pin(a)
    c.prepare([0, 1, 2, 3, 4, 5])
    before_tables = [t.copy() for t in c.host_tables()]
    before = c.stats()
    with pytest.raises(B.LoraError) as e:
        c.prepare([6, 9])  # 6 fits after evicting 1; 9 (rank 32) finds no two adjacent free units
    assert e.value.status == -6 and "fragmented" in B.load().lora_last_error().decode()
    assert resident(c) == {0, 1, 2, 3, 4, 5}
    after = c.stats()
    assert after == before
    for t0, t1 in zip(before_tables, c.host_tables()):
        assert np.array_equal(t0, t1)
    c.prepare([6])
    st = c.stats()
    assert st["misses"] == before["misses"] + 1 and st["hits"] == before["hits"]
    assert st["bytes_copied"] == before["bytes_copied"] + 2 * 16 * (D_IN + D_OUT)
    assert 6 in resident(c) and st["evictions"] == before["evictions"] + 1


def test_rejections():
    lib = B.load()
    h = ctypes.c_void_p()
    tab = lib.lora_cache_table_bytes(4)
    assert lib.lora_cache_create(BASE + 16, tab + 4096, 4, 1, 64, 64, B.LORA_CACHE_DRY, ctypes.byref(h)) == -4
    assert lib.lora_cache_create(BASE, tab, 4, 1, 64, 64, B.LORA_CACHE_DRY, ctypes.byref(h)) == -6
    assert lib.lora_cache_create(BASE, tab + 4096, 4, 7, 64, 64, B.LORA_CACHE_DRY, ctypes.byref(h)) == -5
    assert lib.lora_cache_create(BASE, tab + 4096, 0, 1, 64, 64, B.LORA_CACHE_DRY, ctypes.byref(h)) == -1
    assert lib.lora_cache_create(BASE, tab + 4096, 4, 1, 64, 64, 6, ctypes.byref(h)) == -1
    c, _ = cache_for(2, n=4)
    with pytest.raises(B.LoraError):
        c.prepare([0, 4])           # id out of range
    with pytest.raises(B.LoraError):
        c.register(1, np.zeros(1, np.uint16), np.zeros(1, np.uint16), 300, 1.0)
    c2 = B.AdapterCache.dry_run(tab + 4 * extent(16), 4, "bf16", D_IN, D_OUT)
    with pytest.raises(B.LoraError) as e:
        c2.prepare([1])             # never registered
    assert e.value.status == -3
    c.prepare([0])
    with pytest.raises(B.LoraError):
        c.register(0, np.zeros(1, np.uint16), np.zeros(1, np.uint16), 16, 1.0)  # resident
    c.prepare([])                   # empty batch: nothing to do
