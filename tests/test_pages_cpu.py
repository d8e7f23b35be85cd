"""Paged adapter storage, host side: the page-count helper and the frame
allocator of a page pool (no GPU).

The allocator is a free list, so it cannot fragment: after any sequence of
takes and gives, a request for at most the free count succeeds, and no frame
is ever handed out twice.  That is the property unified paging exists for
("Multi-LoRA Serving in Production ..." (llms.blog), section "Unified Paged
Memory"), checked here against a brute-force model of which frames are free.
"""

import numpy as np
import pytest

from segmented_gather_gemm_lora_amd import binding as B


@pytest.fixture(scope="module", autouse=True)
def _lib():
    B.load()


@pytest.mark.parametrize("nbytes,page,want", [
    (0, 64, 0), (1, 64, 1), (64, 64, 1), (65, 64, 2),
    (16 * 4096 * 2, 16384, 8),          # rank-16 A of a 4096-wide projection, 16 KB pages
    (14336 * 64 * 2, 65536, 28),        # rank-64 B of a 14336-wide projection, 64 KB pages
    (3 * 1000 * 4, 256, 47),            # fp32 [3, 1000]: 12000 B over 256 B pages
])
def test_pages_needed(nbytes, page, want):
    assert B.lora_pages_needed(nbytes, page) == want


@pytest.mark.parametrize("nbytes,page", [(-1, 64), (10, 0), (10, 32), (10, 96), (10, 3 << 10), (10, 1 << 25)])
def test_pages_needed_rejects(nbytes, page):
    assert B.lora_pages_needed(nbytes, page) == -1


def test_fresh_allocator_order_and_lifo():
    a = B.PageAlloc(10)
    assert a.free == 10
    f = a.take(4)
    assert list(f) == [0, 1, 2, 3]
    a.give([2, 0])
    assert a.free == 8
    # last given is taken first
    assert list(a.take(2)) == [0, 2]
    assert list(a.take(1)) == [4]
    a.close()


def test_take_all_or_nothing():
    a = B.PageAlloc(5)
    a.take(3)
    with pytest.raises(B.LoraError) as e:
        a.take(3)
    assert e.value.status == -6  # LORA_ERR_WORKSPACE
    assert a.free == 2
    assert len(a.take(2)) == 2 and a.free == 0
    assert len(a.take(0)) == 0


@pytest.mark.parametrize("bad", [[7], [-1], [1, 1], [2, 9]])
def test_give_rejects_and_changes_nothing(bad):
    a = B.PageAlloc(8)
    a.take(4)  # frames 0..3 taken
    with pytest.raises(B.LoraError) as e:
        a.give(bad)
    assert e.value.status == -1
    assert a.free == 4
    # the taken frames are all still taken: giving them back works once
    a.give([0, 1, 2, 3])
    assert a.free == 8


def test_create_rejects():
    with pytest.raises(B.LoraError):
        B.PageAlloc(0)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_no_fragmentation_random_sequence(seed):
    """Random adapters of mixed ranks come and go; every request that fits the
    free count succeeds and frames are unique among live allocations."""
    rng = np.random.default_rng(seed)
    n_frames = 500
    a = B.PageAlloc(n_frames)
    live = {}
    free = set(range(n_frames))
    for step in range(400):
        if live and (rng.random() < 0.45 or len(free) < 40):
            k = list(live)[rng.integers(len(live))]
            fr = live.pop(k)
            a.give(fr[rng.permutation(len(fr))])
            free |= set(fr.tolist())
        else:
            # a mix like the pages' rank range: A and B of a rank-r adapter, 16 KB pages
            r = int(rng.choice([8, 16, 32, 64]))
            n = B.lora_pages_needed(r * 4096 * 2, 16384) + B.lora_pages_needed(4096 * r * 2, 16384)
            if n > len(free):
                with pytest.raises(B.LoraError):
                    a.take(n)
                continue
            fr = a.take(n)
            assert len(set(fr.tolist())) == n
            assert set(fr.tolist()) <= free
            free -= set(fr.tolist())
            live[step] = fr
        assert a.free == len(free)
    a.close()


def test_paged_call_argument_errors():
    """The paged calls check pages and page_bytes (and then everything the dense
    calls check) before any GPU work."""
    from test_abi_cpu import FX, HostPlan, _valid_plan

    L = B.load()
    plan = _valid_plan()
    need = B.lora_workspace_bytes(B.LORA_OP_SGMV, 8, 256, 256, 8)
    sg = L.lora_sgmv_paged
    for page, st in [(0, -1), (32, -1), (100, -1), (1 << 25, -1)]:
        assert sg(None, 1, FX, 256, 256, plan.dev(), FX, page, FX, 256, 256, FX, need) == st
    assert sg(None, 1, FX, 256, 256, plan.dev(), None, 16384, FX, 256, 256, FX, need) == -1
    assert sg(None, 1, FX, 256, 256, plan.dev(), FX + 8, 16384, FX, 256, 256, FX, need) == -4
    assert sg(None, 1, FX, 256, 256, plan.dev(), FX, 16384, FX, 256, 256, FX, need - 1) == -6
    assert sg(None, 9, FX, 256, 256, plan.dev(), FX, 16384, FX, 256, 256, FX, need) == -5
    empty = HostPlan(0)
    assert B.lora_build_segments(0, None, 0, None, None, None, None, empty.seg) == 0
    assert sg(None, 1, None, 0, 0, empty.dev(None), FX, 16384, None, 0, 0, None, 0) == 0
    bg = L.lora_bgmv_paged
    needb = B.lora_workspace_bytes(B.LORA_OP_BGMV, 64, 4096, 4096, 16)
    assert bg(None, 1, 64, FX, 4096, 4096, FX, FX, FX, FX, FX, 32, 16, FX, 48, FX, 4096, 4096, FX, needb) == -1
    assert bg(None, 1, 64, FX, 4096, 4096, FX, FX, FX, FX, FX, 32, 16, None, 16384, FX, 4096, 4096, FX,
              needb) == -1
    assert bg(None, 1, 64, FX, 4096, 4096, FX, FX, FX, FX, FX, 32, 300, FX, 16384, FX, 4096, 4096, FX,
              needb) == -2
    assert bg(None, 1, 64, FX, 4096, 4096, FX, FX, FX, FX, FX, 32, 16, FX, 16384, FX, 4096, 4096, FX,
              needb - 1) == -6
    assert bg(None, 1, 0, None, 0, 0, None, None, None, None, None, 0, 16, FX, 16384, None, 0, 0, None, 0) == 0
    w = L.lora_pages_write
    assert w(None, FX, 16384, FX, FX, 0) == 0          # nothing to copy
    assert w(None, FX, 1000, FX, FX, 64) == -1         # page size
    assert w(None, None, 16384, FX, FX, 64) == -1
    assert w(None, FX, 16384, None, FX, 64) == -1
    assert w(None, FX, 16384, FX, FX + 4, 64) == -4    # source alignment
    assert w(None, FX, 16384, FX, FX, -1) == -1
