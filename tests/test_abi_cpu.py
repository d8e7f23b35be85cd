"""The C-ABI library on the CPU: it loads, exports what the header declares,
builds segments identical to the oracle's brute-force segments, and rejects bad
arguments from the host before any GPU call."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from segmented_gather_gemm_lora_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora_mi355x.h")

FAKE_BASE = 0x7F0000000000  # plan building never dereferences device addresses


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_header_function():
    lib = B.load()
    names = header_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTS) == names
    assert "gfx950" in B.lora_version()


def test_status_strings():
    for code, name in B.STATUS.items():
        assert B.lora_status_string(code) == name
    assert B.lora_status_string(-99) == "LORA_ERR_UNKNOWN"


@pytest.mark.parametrize("r,d_in,d_out", [(16, 8192, 8192), (8, 4096, 14336), (1, 1, 1), (256, 4096, 12288),
                                          (0, 5, 5)])
def test_adapter_numel_matches_oracle(r, d_in, d_out):
    assert B.lora_adapter_numel(r, d_in, d_out) == oracle.adapter_numel(r, d_in, d_out)


def test_adapter_numel_negative():
    assert B.lora_adapter_numel(-1, 3, 3) == -1


class HostPlan:
    """Segments built into plain host memory (numpy, bound with
    lora_segments_bind), read back through the header layout and the struct."""

    def __init__(self, capacity):
        self.capacity = capacity
        self.nbytes = B.lora_segments_bytes(capacity)
        self.raw = np.zeros((self.nbytes + 32) // 8, dtype=np.uint64)
        self.off = (-self.raw.ctypes.data) % 16  # 16-byte aligned start
        self.h = B.LoraSegments()
        assert B.lora_segments_bind(self.ptr, capacity, ctypes.addressof(self.h)) == 0
        self._devs = []

    @property
    def ptr(self):
        return self.raw.ctypes.data + self.off

    @property
    def seg(self):
        return ctypes.addressof(self.h)

    def dev(self, buf=FAKE_BASE + 0x1000000, host=None):
        """Address of a device-style struct for argument checks (no GPU call):
        the host copy is this buffer (or `host`), the device buffer `buf`."""
        d = B.LoraSegments()
        ctypes.memmove(ctypes.addressof(d), ctypes.addressof(self.h), ctypes.sizeof(d))
        d.buf = buf
        d.host = self.ptr if host is None else host
        self._devs.append(d)
        return ctypes.addressof(d)

    def _u8(self):
        return self.raw.view(np.uint8)[self.off: self.off + self.nbytes]

    def header(self):
        h = B.plan_header(self._u8())
        return dict(magic=h["magic"], T=h["num_tokens"], Tp=h["num_sorted"], S=h["num_segments"],
                    nblk=h["num_blocks"], max_rank=h["max_rank"], max_len=h["max_len"], seg=h["seg_offset"],
                    blk=h["blk_offset"], perm=h["perm_offset"], used=h["bytes_used"], nchunk=h["num_chunks"],
                    chunk=h["chunk_offset"])

    def arrays(self):
        h = B.plan_header(self._u8())
        a = B.plan_arrays(self._u8(), h)
        return a["desc"], a["blocks"], a["perm"], a["chunks"]

    def tail(self):
        h = B.plan_header(self._u8())
        a = B.plan_arrays(self._u8(), h)
        return a["unadapted"], a["segidx"], h

    def table(self):
        return B.segment_table(self.h)


def make_tables(N, rng, ranks=None):
    if ranks is None:
        ranks = rng.integers(1, 257, N).astype(np.int32)
    ranks = np.asarray(ranks, dtype=np.int32)
    alpha = rng.uniform(0.5, 64, N).astype(np.float32)
    A = (FAKE_BASE + 4096 * np.arange(N, dtype=np.uint64) * 2).astype(np.uint64)
    Bt = (A + np.uint64(4096)).astype(np.uint64)
    return A, Bt, ranks, alpha


def build(ids, N, A, Bt, ranks, alpha, plan=None):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    plan = plan or HostPlan(len(ids))
    st = B.lora_build_segments(len(ids), ids.ctypes.data if len(ids) else None, N, A.ctypes.data, Bt.ctypes.data,
                               ranks.ctypes.data, alpha.ctypes.data, plan.seg)
    return st, plan


@pytest.mark.parametrize("T,N,none_p,seed", [(0, 3, 0.0, 0), (1, 1, 0.0, 1), (8, 2, 0.0, 2), (64, 32, 0.0, 3),
                                             (200, 9, 0.3, 4), (1000, 3, 0.1, 5), (4096, 1000, 0.0, 6),
                                             (50, 4, 1.0, 7)])
def test_plan_matches_oracle_segments(T, N, none_p, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, N, T).astype(np.int32)
    ids[rng.random(T) < none_p] = -1
    A, Bt, ranks, alpha = make_tables(N, rng)
    st, plan = build(ids, N, A, Bt, ranks, alpha)
    assert st == 0, B.last_error()
    perm_o, indptr_o, adapter_o = oracle.segments(ids, N)
    h = plan.header()
    desc, blk, perm, chunks = plan.arrays()
    assert h["magic"] == B.PLAN_MAGIC and h["T"] == T and h["Tp"] == len(perm_o)
    assert h["S"] == len(adapter_o)
    assert np.array_equal(perm, perm_o)
    assert np.array_equal(desc["adapter"], adapter_o)
    assert np.array_equal(desc["start"], indptr_o[:-1])
    assert np.array_equal(desc["len"], np.diff(indptr_o))
    assert np.array_equal(desc["rank"], ranks[adapter_o])
    assert np.array_equal(desc["A"], A[adapter_o]) and np.array_equal(desc["B"], Bt[adapter_o])
    # the segment table of the struct (the boundary's outputs)
    t = plan.table()
    assert plan.h.num_segments == len(adapter_o) and plan.h.num_tokens == len(perm_o) and plan.h.batch_tokens == T
    assert plan.h.max_rank == (int(ranks[adapter_o].max()) if len(adapter_o) else 0)
    assert np.array_equal(t["perm"], perm_o) and np.array_equal(t["seg_indptr"], indptr_o)
    assert np.array_equal(t["seg_adapter"], adapter_o) and np.array_equal(t["seg_rank"], ranks[adapter_o])
    assert np.array_equal(t["seg_A"], A[adapter_o]) and np.array_equal(t["seg_B"], Bt[adapter_o])
    assert np.array_equal(t["seg_scale"], (alpha[adapter_o] / ranks[adapter_o].astype(np.float32)).astype(np.float32))
    # scale = alpha / rank in fp32 (correctly rounded division)
    assert np.array_equal(desc["scale"], (alpha[adapter_o] / ranks[adapter_o].astype(np.float32)).astype(np.float32))
    nb = (np.diff(indptr_o) + 15) // 16
    assert h["nblk"] == int(nb.sum())
    assert np.array_equal(desc["blk0"], np.concatenate([[0], np.cumsum(nb)[:-1]]).astype(np.int32) if len(nb) else [])
    # block descriptors: segment, adapter fields copied, 16-row windows of perm
    seg_of_blk = np.repeat(np.arange(len(nb)), nb)
    assert np.array_equal(blk["seg"], seg_of_blk)
    assert h["blk"] % 128 == 0
    for b, sgi in enumerate(seg_of_blk):
        d = desc[sgi]
        q0 = 16 * (b - d["blk0"])
        n = min(16, d["len"] - q0)
        assert blk["n"][b] == n and blk["p0"][b] == d["start"] + q0
        assert blk["A"][b] == d["A"] and blk["B"][b] == d["B"] and blk["rank"][b] == d["rank"]
        assert blk["scale"][b] == d["scale"]
        assert blk["rows"][b][:n].tolist() == perm_o[d["start"] + q0: d["start"] + q0 + n].tolist()
        assert (blk["rows"][b][n:] == -1).all()
    # chunks: consecutive runs of up to 4 blocks (64 rows) inside one segment, covering every row once
    want = [(si, int(d["blk0"]) + i, min(4, int(nbs) - i)) for si, (d, nbs) in enumerate(zip(desc, nb))
            for i in range(0, int(nbs), 4)]
    assert h["nchunk"] == len(want) and h["chunk"] % 64 == 0
    for ch, (si, fb, cnt) in zip(chunks, want):
        d = desc[si]
        q0 = 16 * (fb - d["blk0"])
        n = min(64, d["len"] - q0)
        assert (ch["seg"], ch["first_blk"], ch["nblk"]) == (si, fb, cnt)
        assert ch["n"] == n and ch["p0"] == d["start"] + q0 and ch["rank"] == d["rank"]
        assert ch["A"] == d["A"] and ch["B"] == d["B"] and ch["scale"] == d["scale"]
        assert ch["rows"][:n].tolist() == perm_o[d["start"] + q0: d["start"] + q0 + n].tolist()
        assert (ch["rows"][n:] == -1).all()
    assert h["max_rank"] == (int(ranks[adapter_o].max()) if len(adapter_o) else 0)
    assert h["used"] <= plan.nbytes
    # tokens without an adapter, in order, after the sorted ones; segment of each sorted position
    rest, segidx, hh = plan.tail()
    assert np.array_equal(rest, np.nonzero(ids < 0)[0])
    assert np.array_equal(segidx, np.repeat(np.arange(len(adapter_o)), np.diff(indptr_o)))
    assert hh["segidx_offset"] % 16 == 0 and hh["segidx_offset"] >= hh["chunk_offset"] + 320 * h["nchunk"]
    S = len(adapter_o)
    assert hh["soa_offset"] % 16 == 0 and hh["soa_offset"] >= hh["segidx_offset"] + 4 * h["Tp"]
    assert hh["bytes_used"] == hh["soa_offset"] + 16 * S + 4 * (S + 1) + 12 * S


def test_plan_errors():
    rng = np.random.default_rng(0)
    A, Bt, ranks, alpha = make_tables(4, rng, ranks=[8, 16, 0, 300])
    ok_ids = np.array([0, 1, 1, -1], dtype=np.int32)
    st, _ = build(ok_ids, 4, A, Bt, ranks, alpha)
    assert st == 0  # unused adapters with bad ranks are not looked at
    assert build([0, 4], 4, A, Bt, ranks, alpha)[0] == -3  # id >= n_adapters
    assert build([0, -2], 4, A, Bt, ranks, alpha)[0] == -3  # id < -1
    assert build([2], 4, A, Bt, ranks, alpha)[0] == -2  # rank 0
    assert build([3], 4, A, Bt, ranks, alpha)[0] == -2  # rank 300
    A2 = A.copy()
    A2[1] += 8
    assert build([1], 4, A2, Bt, ranks, alpha)[0] == -4  # misaligned adapter address
    small = HostPlan(2)
    assert build(ok_ids, 4, A, Bt, ranks, alpha, plan=small)[0] == -6  # batch larger than the capacity
    assert "ids[1]" in (build([0, 9], 4, A, Bt, ranks, alpha)[0] and B.last_error())
    plan = HostPlan(4)
    lib = B.load()
    assert lib.lora_build_segments(3, None, 4, A.ctypes.data, Bt.ctypes.data, ranks.ctypes.data, alpha.ctypes.data,
                                   plan.seg) == -1  # NULL ids
    assert lib.lora_build_segments(-1, None, 4, None, None, None, None, plan.seg) == -1
    assert lib.lora_build_segments(2, ok_ids.ctypes.data, 4, None, None, None, None, plan.seg) == -1
    assert lib.lora_build_segments(2, ok_ids.ctypes.data, 4, A.ctypes.data, Bt.ctypes.data, ranks.ctypes.data,
                                   alpha.ctypes.data, None) == -1  # no struct
    unbound = B.LoraSegments()
    assert lib.lora_build_segments(2, ok_ids.ctypes.data, 4, A.ctypes.data, Bt.ctypes.data, ranks.ctypes.data,
                                   alpha.ctypes.data, ctypes.addressof(unbound)) == -1  # not bound
    s2 = B.LoraSegments()
    assert lib.lora_segments_bind(plan.ptr + 4, 4, ctypes.addressof(s2)) == -4  # misaligned buffer
    assert lib.lora_segments_bind(None, 4, ctypes.addressof(s2)) == -1
    assert lib.lora_segments_bind(plan.ptr, -1, ctypes.addressof(s2)) == -1
    # upload checks before any copy: unbound device struct, the same buffer twice, too small a device buffer
    st, full = build(ok_ids, 4, A, Bt, ranks, alpha)
    assert st == 0
    assert lib.lora_segments_upload(full.seg, ctypes.addressof(unbound), None) == -1
    same = B.LoraSegments()
    assert lib.lora_segments_bind(full.ptr, 4, ctypes.addressof(same)) == 0
    assert lib.lora_segments_upload(full.seg, ctypes.addressof(same), None) == -1
    tiny = B.LoraSegments()
    assert lib.lora_segments_bind(FX, 1, ctypes.addressof(tiny)) == 0
    assert lib.lora_segments_upload(full.seg, ctypes.addressof(tiny), None) == -6
    assert lib.lora_segments_upload(None, ctypes.addressof(tiny), None) == -1


def _valid_plan(T=8, N=2, rank=8):
    rng = np.random.default_rng(1)
    A, Bt, ranks, alpha = make_tables(N, rng, ranks=[rank] * N)
    ids = rng.integers(0, N, T).astype(np.int32)
    st, plan = build(ids, N, A, Bt, ranks, alpha)
    assert st == 0
    return plan


FX = 0x7F1000000000  # fake 16-byte-aligned device pointers: validation fails before any use


def test_sgmv_argument_errors():
    plan = _valid_plan()
    empty = HostPlan(0)
    assert B.lora_build_segments(0, None, 0, None, None, None, None, empty.seg) == 0
    sh = B.lora_sgmv_shrink
    # bad dtype
    assert sh(None, 7, FX, 256, 256, plan.dev(), FX, 8, None, 0) == -5
    # NULL plan / plan without magic
    assert sh(None, 1, FX, 256, 256, None, FX, 8, None, 0) == -1
    junk = np.zeros(64, dtype=np.uint64)
    assert sh(None, 1, FX, 256, 256, plan.dev(host=junk.ctypes.data), FX, 8, None, 0) == -8
    # an empty batch is a successful no-op, even with NULL buffers
    assert sh(None, 1, None, 0, 0, empty.dev(None), None, 0, None, 0) == 0
    assert B.lora_sgmv_expand(None, 1, None, 0, empty.dev(None), None, 0, 0, None, 0) == 0
    # NULL x, v, device buffer of the segments
    assert sh(None, 1, None, 256, 256, plan.dev(), FX, 8, None, 0) == -1
    assert sh(None, 1, FX, 256, 256, plan.dev(), None, 8, None, 0) == -1
    assert sh(None, 1, FX, 256, 256, plan.dev(None), FX, 8, None, 0) == -1
    # ldv smaller than the plan's max rank; ldv not a multiple of 4; v misaligned
    assert sh(None, 1, FX, 256, 256, plan.dev(), FX, 4, None, 0) == -2
    assert sh(None, 1, FX, 256, 256, plan.dev(), FX, 10, None, 0) == -4
    assert sh(None, 1, FX, 256, 256, plan.dev(), FX + 4, 8, None, 0) == -4
    # x not aligned to its element size; ldx < d_in; d_in < 1
    assert sh(None, 1, FX + 1, 256, 256, plan.dev(), FX, 8, None, 0) == -4
    assert sh(None, 1, FX, 100, 256, plan.dev(), FX, 8, None, 0) == -1
    assert sh(None, 1, FX, 256, 0, plan.dev(), FX, 8, None, 0) == -1
    ex = B.lora_sgmv_expand
    assert ex(None, 1, FX, 8, plan.dev(), None, 256, 256, None, 0) == -1
    assert ex(None, 1, FX, 8, plan.dev(), FX, 100, 256, None, 0) == -1
    assert ex(None, 0, FX, 8, plan.dev(), FX + 2, 256, 256, None, 0) == -4  # f32 y misaligned
    assert ex(None, 1, FX, 2, plan.dev(), FX, 256, 256, None, 0) == -2


def test_bgmv_argument_errors():
    sh = B.lora_bgmv_shrink
    ex = B.lora_bgmv_expand
    assert sh(None, 1, 0, None, 0, 0, None, None, None, 0, 16, None, 0, None, 0) == 0  # T = 0
    assert sh(None, 1, -1, FX, 64, 64, FX, FX, FX, 4, 16, FX, 16, None, 0) == -1
    assert sh(None, 1, 70000, FX, 64, 64, FX, FX, FX, 4, 16, FX, 16, None, 0) == -1
    assert sh(None, 1, 4, FX, 64, 64, FX, FX, FX, 4, 0, FX, 16, None, 0) == -2
    assert sh(None, 1, 4, FX, 64, 64, FX, FX, FX, 4, 257, FX, 16, None, 0) == -2
    assert sh(None, 1, 4, FX, 64, 64, None, FX, FX, 4, 16, FX, 16, None, 0) == -1
    assert sh(None, 1, 4, FX, 64, 64, FX, FX, FX, 4, 16, FX, 8, None, 0) == -2
    assert sh(None, 3, 4, FX, 64, 64, FX, FX, FX, 4, 16, FX, 16, None, 0) == -5
    assert ex(None, 1, 0, None, 0, None, None, None, None, 0, 16, None, 0, 0, None, 0) == 0
    assert ex(None, 1, 4, FX, 16, FX, FX, FX, None, 4, 16, FX, 64, 64, None, 0) == -1
    assert ex(None, 1, 4, FX, 16, FX, FX, FX, FX, 4, 16, FX, 32, 64, None, 0) == -1


def test_fused_argument_errors():
    plan = _valid_plan()
    f = B.lora_fused_linear
    assert f(None, 0, FX, 256, 256, FX, 256, plan.dev(), FX, 256, FX, 1 << 20) == -5  # f32 not offered
    assert f(None, 1, FX, 256, 256, FX, 256, plan.dev(), FX, 256, FX, 16) == -6  # workspace too small
    assert f(None, 1, FX, 256, 256, FX, 256, plan.dev(), FX, 256, None, 1 << 20) == -6
    assert f(None, 1, FX + 2, 256, 256, FX, 256, plan.dev(), FX, 256, FX, 1 << 20) == -4
    assert f(None, 1, None, 256, 256, FX, 256, plan.dev(), FX, 256, FX, 1 << 20) == -1
    need = B.lora_workspace_bytes(B.LORA_OP_FUSED, 8, 256, 256, 8)
    assert need >= 8 * 16 * 4


def test_fused_e4m3_argument_errors():
    """The FP8-base entry: the scale must be finite and non-zero, d_in a
    multiple of 16; otherwise the bf16 entry's rules."""
    plan = _valid_plan()
    f = B.lora_fused_linear_e4m3
    ok = 1 << 20
    for bad in (0.0, float("inf"), float("-inf"), float("nan")):
        assert f(None, FX, 256, 256, FX, bad, 256, plan.dev(), FX, 256, FX, ok) == -1, bad
    assert f(None, FX, 264, 264, FX, 0.5, 256, plan.dev(), FX, 256, FX, ok) == -4  # d_in % 16 = 8
    assert f(None, FX, 256, 256, FX + 8, 0.5, 256, plan.dev(), FX, 256, FX, ok) == -4  # W0 not 16-byte aligned
    assert f(None, FX, 256, 256, FX, 0.5, 256, plan.dev(), FX, 256, FX, 16) == -6  # workspace too small
    assert f(None, FX, 256, 256, None, 0.5, 256, plan.dev(), FX, 256, FX, ok) == -1
    empty = HostPlan(0)
    assert B.lora_build_segments(0, None, 0, None, None, None, None, empty.seg) == 0
    assert f(None, None, 0, 256, None, 0.5, 256, empty.dev(None), None, 256, None, 0) == 0  # T = 0


def test_combined_argument_errors():
    plan = _valid_plan()
    sg = B.lora_sgmv
    need = B.lora_workspace_bytes(B.LORA_OP_SGMV, 8, 256, 256, 8)
    assert need >= 8 * 8 * 4
    assert sg(None, 1, FX, 256, 256, plan.dev(), FX, 256, 256, FX, need - 1) == -6
    assert sg(None, 1, FX, 256, 256, plan.dev(), FX, 256, 256, None, need) == -6
    assert sg(None, 1, FX, 256, 256, plan.dev(), FX, 256, 256, FX + 8, need) == -4
    assert sg(None, 1, None, 256, 256, plan.dev(), FX, 256, 256, FX, need) == -1
    assert sg(None, 1, FX, 256, 256, plan.dev(), None, 256, 256, FX, need) == -1
    assert sg(None, 9, FX, 256, 256, plan.dev(), FX, 256, 256, FX, need) == -5
    empty = HostPlan(0)
    assert B.lora_build_segments(0, None, 0, None, None, None, None, empty.seg) == 0
    assert sg(None, 1, None, 0, 0, empty.dev(None), None, 0, 0, None, 0) == 0
    bg = B.lora_bgmv
    needb = B.lora_workspace_bytes(B.LORA_OP_BGMV, 64, 4096, 4096, 16)
    # a 256 B status block in front of the fp32 partial sums of 4 d_in slices
    # (the two-kernel form), then the same sums as tagged 64-bit words (the
    # one-launch form)
    part = 4 * 64 * 16 * 4 + 256
    assert needb == 256 + 3 * part
    assert bg(None, 1, 0, None, 0, 0, None, None, None, None, None, 0, 16, None, 0, 0, None, 0) == 0
    assert bg(None, 1, 64, FX, 4096, 4096, FX, FX, FX, FX, FX, 32, 16, FX, 4096, 4096, FX, needb - 1) == -6
    assert bg(None, 1, 64, FX, 4096, 4096, FX, FX, None, FX, FX, 32, 16, FX, 4096, 4096, FX, needb) == -1
    assert bg(None, 1, 64, FX, 4096, 4096, FX, FX, FX, FX, FX, 32, 300, FX, 4096, 4096, FX, needb) == -2
    assert bg(None, 1, 64, FX, 4096, 4096, FX, FX, FX, FX, FX, 32, 16, FX, 100, 4096, FX, needb) == -1


def test_grouped_bgmv_host_checks():
    """Grouped BGMV: the workspace is the 256-byte status block plus, per
    projection, three times its 256-byte rounded region of fp32 partial sums
    (those sums, then the one-launch form's 8-byte tagged words), and malformed
    calls are rejected before any GPU work."""
    import ctypes as C

    projs = (B.LoraProj * 3)()
    for p, (d_in, d_out, r) in enumerate([(4096, 4096, 16), (4096, 1024, 8), (4096, 1024, 64)]):
        projs[p] = B.LoraProj(FX, FX + 0x100000 * (p + 1), FX, FX, FX, FX, d_in, d_out, d_in, d_out, r, 0)
    def partials(T, d_in, r):  # fp32 partial sums over at most 4 slices of 256+ elements of d_in, plus slack
        return min((d_in + 255) // 256, 4) * T * ((r + 3) // 4 * 4) * 4 + 256

    want = 256 + sum(3 * ((partials(64, d_in, r) + 255) // 256 * 256)
                     for d_in, d_out, r in [(4096, 4096, 16), (4096, 1024, 8), (4096, 1024, 64)])
    ptr = C.cast(projs, C.c_void_p)
    assert B.lora_bgmv_grouped_workspace_bytes(64, ptr, 3) == want
    assert B.lora_bgmv_grouped_workspace_bytes(64, ptr, 0) == 0
    assert B.lora_bgmv_grouped_workspace_bytes(64, None, 3) == 0
    g = B.lora_bgmv_grouped
    assert g(None, 1, 64, FX, 32, ptr, 9, FX, want) == -1          # too many projections
    assert g(None, 1, 64, FX, 32, None, 3, FX, want) == -1         # no projections
    assert g(None, 1, -1, FX, 32, ptr, 3, FX, want) == -1          # negative T
    assert g(None, 1, 64, FX, 32, ptr, 3, FX, want - 16) == -6     # workspace too small
    assert g(None, 1, 64, None, 32, ptr, 3, FX, want) == -1        # no ids
    assert g(None, 1, 64, FX, 32, ptr, 3, FX + 4, want) == -4      # misaligned workspace
    projs[2].max_rank = 0
    assert g(None, 1, 64, FX, 32, ptr, 3, FX, want) == -2
    projs[2].max_rank = 64
    projs[1].y = projs[0].y
    assert g(None, 1, 64, FX, 32, ptr, 3, FX, want) == -1          # two projections write one y
    projs[1].y = FX + 0x200000
    projs[1].d_in = 0
    assert g(None, 1, 64, FX, 32, ptr, 3, FX, want) == -1          # d_in < 1
    assert g(None, 1, 0, FX, 32, ptr, 3, None, 0) in (0, -1)       # T = 0: nothing to do (or the d_in error)


def test_workspace_bytes():
    for op in (0, 1, 2, 3):
        assert B.lora_workspace_bytes(op, 4096, 4096, 4096, 16) == 0
    assert B.lora_workspace_bytes(99, 1, 1, 1, 1) == ctypes.c_size_t(-1).value


def test_header_is_a_c_abi(tmp_path):
    """tests/c/abi_c_check.c, built as C99 with gcc against the header and
    linked with the library, runs the host-only entry points."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    lib = B.lib_path()
    exe = str(tmp_path / "abi_c_check")
    src = os.path.join(ROOT, "tests", "c", "abi_c_check.c")
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), src, "-o", exe, lib,
                    "-Wl,-rpath," + os.path.dirname(lib)], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True)
    assert out.stdout.strip() == "ok"


def test_grouped_sgmv_host_checks():
    """Grouped SGMV: workspace = the projections' 256-byte rounded regions;
    malformed calls are rejected before any GPU work."""
    L = B.load()
    plan = _valid_plan()  # T = 8, max rank 8
    projs = (B.LoraSgmvProj * 2)()
    for p in range(2):
        projs[p] = B.LoraSgmvProj(FX, FX + 0x100000 * (p + 1), plan.dev(), 256, 256, 256, 256)
    one = min((256 + 255) // 256, 4) * 8 * 8 * 4 + 256  # fp32 partial sums of the d_in slices, plus slack
    need = L.lora_sgmv_grouped_workspace_bytes(projs, 2)
    assert need == 2 * ((one + 255) // 256 * 256)
    assert L.lora_sgmv_grouped_workspace_bytes(projs, 0) == 0
    assert L.lora_sgmv_grouped_workspace_bytes(projs, 9) == 0
    g = L.lora_sgmv_grouped
    assert g(None, 1, projs, 2, FX, need - 1) == -6
    assert g(None, 1, projs, 2, FX + 8, need) == -4
    assert g(None, 1, projs, 0, FX, need) == -1
    assert g(None, 1, None, 2, FX, need) == -1
    assert g(None, 9, projs, 2, FX, need) == -5
    projs[1].y = projs[0].y
    assert g(None, 1, projs, 2, FX, need) == -1          # same y twice
    projs[1].y = FX + 0x300000
    projs[1].x = None
    assert g(None, 1, projs, 2, FX, need) == -1          # NULL x
    projs[1].x = FX
    projs[1].seg = None
    assert g(None, 1, projs, 2, FX, need) != 0           # no plan


def test_grouped_sgmv_all_empty_is_noop():
    """Projections whose plans hold no adapted token: nothing to do, no
    workspace needed, no GPU call."""
    L = B.load()
    empty = HostPlan(0)
    assert B.lora_build_segments(0, None, 0, None, None, None, None, empty.seg) == 0
    projs = (B.LoraSgmvProj * 2)()
    for p in range(2):
        projs[p] = B.LoraSgmvProj(None, FX + 0x100000 * (p + 1), empty.dev(None), 256, 256, 256, 256)
    assert L.lora_sgmv_grouped(None, 1, projs, 2, None, 0) == 0
