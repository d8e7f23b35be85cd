"""ctypes binding of liblora_mi355x.so.

Argument marshalling only: every step of the adapter path (plan building,
shrink, expand, the fused layer) runs inside the library.  PyTorch is used for
device memory, pinned host memory and streams.  If the library has not been
built, every entry point raises -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import threading
from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import build as _build

LORA_F32 = 0
LORA_BF16 = 1
DTYPES = {"f32": LORA_F32, "bf16": LORA_BF16}

LORA_OP_SGMV_SHRINK = 0
LORA_OP_SGMV_EXPAND = 1
LORA_OP_BGMV_SHRINK = 2
LORA_OP_BGMV_EXPAND = 3
LORA_OP_FUSED = 4
LORA_OP_SGMV = 5
LORA_OP_BGMV = 6

STATUS = {
    0: "LORA_OK", -1: "LORA_ERR_ARG", -2: "LORA_ERR_RANK", -3: "LORA_ERR_ADAPTER_ID",
    -4: "LORA_ERR_ALIGN", -5: "LORA_ERR_DTYPE", -6: "LORA_ERR_WORKSPACE", -7: "LORA_ERR_HIP",
    -8: "LORA_ERR_PLAN",
}

# Every symbol the public header declares.
EXPORTS = [
    "lora_segments_bytes", "lora_segments_bind", "lora_build_segments", "lora_segments_upload", "lora_sgmv_shrink",
    "lora_sgmv_expand", "lora_sgmv", "lora_bgmv_shrink", "lora_bgmv_expand", "lora_bgmv", "lora_fused_linear", "lora_fused_linear_e4m3",
    "lora_workspace_bytes", "lora_adapter_numel", "lora_status_string", "lora_last_error",
    "lora_version", "lora_profile_launches", "lora_profile_launches_used", "lora_bgmv_grouped",
    "lora_bgmv_grouped_workspace_bytes", "lora_cache_table_bytes", "lora_cache_create", "lora_cache_destroy",
    "lora_cache_register", "lora_cache_pin", "lora_cache_prepare", "lora_cache_view_get", "lora_cache_stats_get",
    "lora_pages_needed", "lora_page_alloc_create", "lora_page_alloc_destroy", "lora_page_alloc_take",
    "lora_page_alloc_give", "lora_page_alloc_free_count", "lora_pages_write", "lora_sgmv_paged", "lora_bgmv_paged",
    "lora_sgmv_grouped", "lora_sgmv_grouped_workspace_bytes", "lora_probe_empty", "lora_probe_stream",
    "lora_probe_chase", "lora_workspace_clear", "lora_debug_wait_limit", "lora_bgmv_noalloc",
]
LORA_CACHE_DRY = 1
MAX_PROJ = 8

PLAN_HEADER_BYTES = 96
CHUNK_BLOCKS = 4
PLAN_MAGIC = 0x4C6F5241
ROW_BLOCK = 16


class LoraError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}: {msg}")
        self.status = status


_i32, _i64, _u64, _vp, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_size_t
_LIB = None
_LOCK = threading.Lock()

_SIGS = {
    "lora_segments_bytes": (_sz, [_i32]),
    "lora_segments_bind": (ctypes.c_int, [_vp, _i32, _vp]),
    "lora_build_segments": (ctypes.c_int, [_i32, _vp, _i32, _vp, _vp, _vp, _vp, _vp]),
    "lora_segments_upload": (ctypes.c_int, [_vp, _vp, _vp]),
    "lora_sgmv_shrink": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _i64, _i32, _vp, _vp, _i64, _vp, _sz]),
    "lora_sgmv_expand": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _i64, _vp, _vp, _i64, _i32, _vp, _sz]),
    "lora_sgmv": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _i64, _i32, _vp, _vp, _i64, _i32, _vp, _sz]),
    "lora_bgmv": (ctypes.c_int, [_vp, ctypes.c_int, _i32, _vp, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                 _vp, _i64, _i32, _vp, _sz]),
    "lora_bgmv_shrink": (ctypes.c_int, [_vp, ctypes.c_int, _i32, _vp, _i64, _i32, _vp, _vp, _vp, _i32, _i32,
                                        _vp, _i64, _vp, _sz]),
    "lora_bgmv_expand": (ctypes.c_int, [_vp, ctypes.c_int, _i32, _vp, _i64, _vp, _vp, _vp, _vp, _i32, _i32,
                                        _vp, _i64, _i32, _vp, _sz]),
    "lora_fused_linear": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _i64, _i32, _vp, _i32, _vp, _vp, _i64, _vp, _sz]),
    "lora_fused_linear_e4m3": (ctypes.c_int, [_vp, _vp, _i64, _i32, _vp, ctypes.c_float, _i32, _vp, _vp, _i64, _vp,
                                              _sz]),
    "lora_workspace_bytes": (_sz, [ctypes.c_int, _i32, _i32, _i32, _i32]),
    "lora_adapter_numel": (_i64, [_i32, _i32, _i32]),
    "lora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "lora_last_error": (ctypes.c_char_p, []),
    "lora_version": (ctypes.c_char_p, []),
    "lora_profile_launches": (ctypes.c_int, [_vp, _vp, _i32]),
    "lora_profile_launches_used": (ctypes.c_int32, []),
    "lora_bgmv_grouped": (ctypes.c_int, [_vp, ctypes.c_int, _i32, _vp, _i32, _vp, _i32, _vp, _sz]),
    "lora_bgmv_grouped_workspace_bytes": (_sz, [_i32, _vp, _i32]),
    "lora_cache_table_bytes": (_sz, [_i32]),
    "lora_cache_create": (ctypes.c_int, [_vp, _sz, _i32, ctypes.c_int, _i32, _i32, ctypes.c_uint, _vp]),
    "lora_cache_destroy": (None, [_vp]),
    "lora_cache_register": (ctypes.c_int, [_vp, _i32, _vp, _vp, _i32, ctypes.c_float]),
    "lora_cache_pin": (ctypes.c_int, [_vp, _i32, ctypes.c_int]),
    "lora_cache_prepare": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp]),
    "lora_cache_view_get": (ctypes.c_int, [_vp, _vp]),
    "lora_cache_stats_get": (ctypes.c_int, [_vp, _vp]),
    "lora_pages_needed": (_i64, [_i64, _i64]),
    "lora_sgmv_grouped": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _i32, _vp, _sz]),
    "lora_sgmv_grouped_workspace_bytes": (_sz, [_vp, _i32]),
    "lora_probe_empty": (ctypes.c_int, [_vp, _i32]),
    "lora_workspace_clear": (ctypes.c_int, [_vp, _vp, _sz]),
    "lora_debug_wait_limit": (ctypes.c_int, [_i32]),
    "lora_bgmv_noalloc": (ctypes.c_int, [_vp, ctypes.c_int, _i32, _vp, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _i32,
                                         _i32, _vp, _i64, _i32]),
    "lora_probe_stream": (ctypes.c_int, [_vp, _vp, _i64, _vp, _i64, _vp, _i32]),
    "lora_probe_chase": (ctypes.c_int, [_vp, _vp, _i32, _vp]),
    "lora_page_alloc_create": (ctypes.c_int, [_i32, _vp]),
    "lora_page_alloc_destroy": (None, [_vp]),
    "lora_page_alloc_take": (ctypes.c_int, [_vp, _i32, _vp]),
    "lora_page_alloc_give": (ctypes.c_int, [_vp, _vp, _i32]),
    "lora_page_alloc_free_count": (_i32, [_vp]),
    "lora_pages_write": (ctypes.c_int, [_vp, _vp, _i64, _vp, _vp, _i64]),
    "lora_sgmv_paged": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _i64, _i32, _vp, _vp, _i64, _vp, _i64, _i32, _vp,
                                       _sz]),
    "lora_bgmv_paged": (ctypes.c_int, [_vp, ctypes.c_int, _i32, _vp, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _i32,
                                       _i32, _vp, _i64, _vp, _i64, _i32, _vp, _sz]),
}


class CacheStats(ctypes.Structure):
    """struct lora_cache_stats."""

    _fields_ = [("batches", _i64), ("hits", _i64), ("misses", _i64), ("evictions", _i64), ("bytes_copied", _i64),
                ("resident_bytes", _i64), ("resident", _i32), ("reserved", _i32)]


class CacheView(ctypes.Structure):
    """struct lora_cache_view."""

    _fields_ = [("pool_A_dev", _vp), ("pool_B_dev", _vp), ("rank_dev", _vp), ("alpha_dev", _vp),
                ("pool_A_host", _vp), ("pool_B_host", _vp), ("rank_host", _vp), ("alpha_host", _vp),
                ("n_adapters", _i32), ("max_rank", _i32)]


assert ctypes.sizeof(CacheStats) == 56 and ctypes.sizeof(CacheView) == 72


class LoraProj(ctypes.Structure):
    """struct lora_proj: one projection of a grouped BGMV call."""

    _fields_ = [("x", _vp), ("y", _vp), ("pool_A_dev", _vp), ("pool_B_dev", _vp), ("pool_rank_dev", _vp),
                ("pool_alpha_dev", _vp), ("ldx", _i64), ("ldy", _i64), ("d_in", _i32), ("d_out", _i32),
                ("max_rank", _i32), ("reserved", _i32)]


assert ctypes.sizeof(LoraProj) == 80


class LoraSegments(ctypes.Structure):
    """struct lora_segments: a batch's segments, bound to a host or device buffer."""

    _fields_ = [("num_segments", _i32), ("num_tokens", _i32), ("max_rank", _i32), ("capacity", _i32),
                ("perm", _vp), ("seg_indptr", _vp), ("seg_adapter", _vp), ("seg_rank", _vp), ("seg_A", _vp),
                ("seg_B", _vp), ("seg_scale", _vp), ("batch_tokens", _i32), ("reserved0", _i32), ("buf", _vp),
                ("host", _vp)]


assert ctypes.sizeof(LoraSegments) == 96


class LoraSgmvProj(ctypes.Structure):
    """struct lora_sgmv_proj: one projection of a grouped SGMV call."""

    _fields_ = [("x", _vp), ("y", _vp), ("seg", _vp), ("ldx", _i64), ("ldy", _i64), ("d_in", _i32), ("d_out", _i32)]


assert ctypes.sizeof(LoraSgmvProj) == 48


def lib_path() -> str:
    return _build.lib_path()


def load():
    """Load the built library (raises if it is missing)."""
    global _LIB
    with _LOCK:
        if _LIB is not None:
            return _LIB
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m segmented_gather_gemm_lora_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
        return lib


def _check(status: int, where: str):
    if status != 0:
        raise LoraError(status, where, load().lora_last_error().decode())


def last_error() -> str:
    return load().lora_last_error().decode()


# ------------------------------------------------------------------ raw C calls (same names)
def lora_segments_bytes(capacity: int) -> int:
    return int(load().lora_segments_bytes(capacity))


def lora_workspace_bytes(op: int, T: int, d_in: int, d_out: int, max_rank: int) -> int:
    return int(load().lora_workspace_bytes(op, T, d_in, d_out, max_rank))


def lora_adapter_numel(r: int, d_in: int, d_out: int) -> int:
    return int(load().lora_adapter_numel(r, d_in, d_out))


def lora_version() -> str:
    return load().lora_version().decode()


def lora_status_string(status: int) -> str:
    return load().lora_status_string(status).decode()


def lora_segments_bind(buf_ptr, capacity, seg_ptr) -> int:
    return int(load().lora_segments_bind(buf_ptr, capacity, seg_ptr))


def lora_build_segments(T, ids_ptr, n_adapters, pool_A_ptr, pool_B_ptr, pool_rank_ptr, pool_alpha_ptr,
                        seg_ptr) -> int:
    return int(load().lora_build_segments(T, ids_ptr, n_adapters, pool_A_ptr, pool_B_ptr, pool_rank_ptr,
                                          pool_alpha_ptr, seg_ptr))


def lora_segments_upload(host_ptr, dev_ptr, stream) -> int:
    return int(load().lora_segments_upload(host_ptr, dev_ptr, stream))


def lora_sgmv_shrink(stream, dtype, x, ldx, d_in, seg, v, ldv, ws, ws_bytes) -> int:
    return int(load().lora_sgmv_shrink(stream, dtype, x, ldx, d_in, seg, v, ldv, ws, ws_bytes))


def lora_sgmv_expand(stream, dtype, v, ldv, seg, y, ldy, d_out, ws, ws_bytes) -> int:
    return int(load().lora_sgmv_expand(stream, dtype, v, ldv, seg, y, ldy, d_out, ws, ws_bytes))


def lora_sgmv(stream, dtype, x, ldx, d_in, seg, y, ldy, d_out, ws, ws_bytes) -> int:
    return int(load().lora_sgmv(stream, dtype, x, ldx, d_in, seg, y, ldy, d_out, ws, ws_bytes))


def lora_bgmv(stream, dtype, T, x, ldx, d_in, ids, pool_A, pool_B, pool_rank, pool_alpha, n_adapters, max_rank,
              y, ldy, d_out, ws, ws_bytes) -> int:
    return int(load().lora_bgmv(stream, dtype, T, x, ldx, d_in, ids, pool_A, pool_B, pool_rank, pool_alpha,
                                n_adapters, max_rank, y, ldy, d_out, ws, ws_bytes))


def lora_bgmv_shrink(stream, dtype, T, x, ldx, d_in, ids, pool_A, pool_rank, n_adapters, max_rank, v, ldv,
                     ws, ws_bytes) -> int:
    return int(load().lora_bgmv_shrink(stream, dtype, T, x, ldx, d_in, ids, pool_A, pool_rank, n_adapters,
                                       max_rank, v, ldv, ws, ws_bytes))


def lora_bgmv_expand(stream, dtype, T, v, ldv, ids, pool_B, pool_rank, pool_alpha, n_adapters, max_rank,
                     y, ldy, d_out, ws, ws_bytes) -> int:
    return int(load().lora_bgmv_expand(stream, dtype, T, v, ldv, ids, pool_B, pool_rank, pool_alpha,
                                       n_adapters, max_rank, y, ldy, d_out, ws, ws_bytes))


def lora_bgmv_grouped(stream, dtype, T, ids, n_adapters, projs, n_proj, ws, ws_bytes) -> int:
    return int(load().lora_bgmv_grouped(stream, dtype, T, ids, n_adapters, projs, n_proj, ws, ws_bytes))


def lora_bgmv_grouped_workspace_bytes(T, projs, n_proj) -> int:
    return int(load().lora_bgmv_grouped_workspace_bytes(T, projs, n_proj))


class _Raw:
    """A raw device address where the calls expect a tensor."""

    def __init__(self, addr):
        self.addr = int(addr or 0)

    def data_ptr(self) -> int:
        return self.addr


class AdapterCache:
    """Residency cache over a device buffer (lora_cache_*): adapters registered
    from pinned host memory are copied in on a copy stream when a batch needs
    them, least recently used ones evicted.  dev_buf: a uint8 device tensor (or
    an int address when dry).  `pool()` gives the tables in the form the
    SGMV/BGMV calls take."""

    def __init__(self, dev_buf, n_adapters: int, dtype: str, d_in: int, d_out: int, dry: bool = False):
        lib = load()
        self._buf = dev_buf  # keeps the device memory alive
        addr = dev_buf if isinstance(dev_buf, int) else _ptr(dev_buf)
        nbytes = self.dry_bytes if isinstance(dev_buf, int) else dev_buf.numel()
        h = ctypes.c_void_p()
        _check(lib.lora_cache_create(addr, nbytes, n_adapters, DTYPES[dtype], d_in, d_out,
                                     LORA_CACHE_DRY if dry else 0, ctypes.byref(h)), "lora_cache_create")
        self.h, self.n_adapters, self.dtype, self.d_in, self.d_out = h, n_adapters, dtype, d_in, d_out
        self.dry = dry
        self._host = {}

    dry_bytes = 0

    @classmethod
    def dry_run(cls, nbytes: int, n_adapters: int, dtype: str, d_in: int, d_out: int):
        """A placement-only cache over a fake 256-byte aligned address range."""
        obj = cls.__new__(cls)
        obj.dry_bytes = nbytes
        cls.__init__(obj, 0x7F0000000000, n_adapters, dtype, d_in, d_out, dry=True)
        return obj

    def close(self):
        if getattr(self, "h", None) is not None and self.h.value:
            load().lora_cache_destroy(self.h)
            self.h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def register(self, adapter: int, A_host, B_host, rank: int, alpha: float):
        """A_host / B_host: host arrays or tensors (pinned for overlapped copies),
        kept referenced by the cache object."""
        self._host[adapter] = (A_host, B_host)
        pa = A_host.ctypes.data if isinstance(A_host, np.ndarray) else A_host.data_ptr()
        pb = B_host.ctypes.data if isinstance(B_host, np.ndarray) else B_host.data_ptr()
        _check(load().lora_cache_register(self.h, adapter, pa, pb, rank, alpha), "lora_cache_register")

    def pin(self, adapter: int, pinned: bool = True):
        _check(load().lora_cache_pin(self.h, adapter, int(pinned)), "lora_cache_pin")

    def prepare(self, ids, copy_stream=None, compute_stream=None):
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        streams = (None, None) if self.dry else (_stream_handle(copy_stream), _stream_handle(compute_stream))
        _check(load().lora_cache_prepare(self.h, ids.ctypes.data if ids.size else None, ids.shape[0], *streams),
               "lora_cache_prepare")

    def stats(self) -> dict:
        st = CacheStats()
        _check(load().lora_cache_stats_get(self.h, ctypes.byref(st)), "lora_cache_stats_get")
        return {f: getattr(st, f) for f, _ in CacheStats._fields_ if f != "reserved"}

    def view(self) -> CacheView:
        v = CacheView()
        _check(load().lora_cache_view_get(self.h, ctypes.byref(v)), "lora_cache_view_get")
        return v

    def pool(self) -> "DevicePool":
        """The current tables as a DevicePool: host mirrors for lora_build_segments,
        device tables for the BGMV calls.  Valid until the next prepare."""
        v = self.view()
        A, Bt, r, a = self.host_tables()
        return DevicePool(storage=self._buf, n_adapters=self.n_adapters, dtype=self.dtype, d_in=self.d_in,
                          d_out=self.d_out, addr_A=A, addr_B=Bt, rank=r, alpha=a, addr_A_dev=_Raw(v.pool_A_dev),
                          addr_B_dev=_Raw(v.pool_B_dev), rank_dev=_Raw(v.rank_dev), alpha_dev=_Raw(v.alpha_dev))

    def host_tables(self):
        """Copies of the host mirrors: (A addresses, B addresses, ranks, alphas)."""
        v, n = self.view(), self.n_adapters
        A = np.ctypeslib.as_array(ctypes.cast(v.pool_A_host, ctypes.POINTER(ctypes.c_uint64)), (n,)).copy()
        Bt = np.ctypeslib.as_array(ctypes.cast(v.pool_B_host, ctypes.POINTER(ctypes.c_uint64)), (n,)).copy()
        r = np.ctypeslib.as_array(ctypes.cast(v.rank_host, ctypes.POINTER(ctypes.c_int32)), (n,)).copy()
        a = np.ctypeslib.as_array(ctypes.cast(v.alpha_host, ctypes.POINTER(ctypes.c_float)), (n,)).copy()
        return A, Bt, r, a


def lora_fused_linear(stream, dtype, x, ldx, d_in, W0, d_out, seg, y, ldy, ws, ws_bytes) -> int:
    return int(load().lora_fused_linear(stream, dtype, x, ldx, d_in, W0, d_out, seg, y, ldy, ws, ws_bytes))


def lora_fused_linear_e4m3(stream, x, ldx, d_in, W0, w0_scale, d_out, seg, y, ldy, ws, ws_bytes) -> int:
    return int(load().lora_fused_linear_e4m3(stream, x, ldx, d_in, W0, w0_scale, d_out, seg, y, ldy, ws, ws_bytes))


def lora_profile_launches(start_events, stop_events, count) -> int:
    return int(load().lora_profile_launches(start_events, stop_events, count))


class KernelTimer:
    """Times the library's next kernel launches with HIP events attached to the
    kernels themselves (hipExtLaunchKernelGGL start/stop events)."""

    _hip = None

    def __init__(self, n: int):
        if KernelTimer._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            KernelTimer._hip = hip
        self.n = n
        self.start = (ctypes.c_void_p * n)()
        self.stop = (ctypes.c_void_p * n)()
        for i in range(n):
            for arr in (self.start, self.stop):
                h = ctypes.c_void_p()
                if KernelTimer._hip.hipEventCreate(ctypes.byref(h)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                arr[i] = h

    def arm(self, first: int, count: int):
        """The next `count` launches record events first .. first+count-1."""
        st = lora_profile_launches(ctypes.addressof(self.start) + 8 * first,
                                   ctypes.addressof(self.stop) + 8 * first, count)
        _check(st, "lora_profile_launches")

    def disarm(self):
        _check(lora_profile_launches(None, None, 0), "lora_profile_launches")

    @staticmethod
    def used() -> int:
        """Launches that took events since the last arm()."""
        return int(load().lora_profile_launches_used())

    def elapsed_us(self, i: int) -> float:
        hip = KernelTimer._hip
        hip.hipEventSynchronize(self.stop[i])
        ms = ctypes.c_float()
        if hip.hipEventElapsedTime(ctypes.byref(ms), self.start[i], self.stop[i]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value * 1e3

    def close(self):
        for i in range(self.n):
            KernelTimer._hip.hipEventDestroy(self.start[i])
            KernelTimer._hip.hipEventDestroy(self.stop[i])


class Prepared:
    """One library call with its arguments converted to C types once, for
    loops that repeat the same call (benchmarks, serving loops): calling the
    object makes the C call and raises on a non-zero status.  `keep` holds
    the tensors whose addresses the arguments carry."""

    __slots__ = ("_fn", "_args", "_name", "_keep")

    def __init__(self, name: str, args, keep=()):
        res, types = _SIGS[name]
        if len(types) != len(args):
            raise TypeError(f"{name} takes {len(types)} arguments, got {len(args)}")
        self._fn = getattr(load(), name)
        self._args = tuple(None if a is None else (a if isinstance(a, ctypes._SimpleCData) else t(a))
                           for t, a in zip(types, args))
        self._name = name
        self._keep = tuple(keep)

    def __call__(self):
        st = self._fn(*self._args)
        if st:
            _check(st, self._name)


# ------------------------------------------------------------------ torch-facing helpers
def _torch():
    import torch

    return torch


def _stream_handle(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def torch_dtype(dtype: str):
    torch = _torch()
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_device(arr: np.ndarray, dtype: str, device="cuda"):
    """Host array (bf16 bit patterns as uint16, or float32) -> device tensor."""
    torch = _torch()
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def to_host_bits(t, dtype: str) -> np.ndarray:
    """Device tensor -> host array in the stored representation."""
    torch = _torch()
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy().astype(np.float32, copy=False)


@dataclass
class DevicePool:
    """Adapters resident in device memory, with their pointer and rank tables."""

    storage: object  # device tensor holding every A_i and B_i (unpadded)
    n_adapters: int
    dtype: str
    d_in: int
    d_out: int
    addr_A: np.ndarray  # uint64 host copies of the tables
    addr_B: np.ndarray
    rank: np.ndarray  # int32
    alpha: np.ndarray  # float32
    addr_A_dev: object = None  # device tables (for BGMV)
    addr_B_dev: object = None
    rank_dev: object = None
    alpha_dev: object = None

    @property
    def max_rank(self) -> int:
        return int(self.rank.max()) if self.rank.size else 0

    @classmethod
    def from_problem(cls, prob, device="cuda") -> "DevicePool":
        torch = _torch()
        storage = to_device(prob.pool, prob.dtype, device)
        base = storage.data_ptr()
        es = prob.esize
        addr_A = (base + prob.a_off.astype(np.uint64) * np.uint64(es)).astype(np.uint64)
        addr_B = (base + prob.b_off.astype(np.uint64) * np.uint64(es)).astype(np.uint64)
        rank = np.ascontiguousarray(prob.ranks, dtype=np.int32)
        alpha = np.ascontiguousarray(prob.alphas, dtype=np.float32)
        p = cls(storage=storage, n_adapters=prob.n_adapters, dtype=prob.dtype, d_in=prob.d_in, d_out=prob.d_out,
                addr_A=addr_A, addr_B=addr_B, rank=rank, alpha=alpha)
        p.addr_A_dev = torch.from_numpy(addr_A.view(np.int64)).to(device)
        p.addr_B_dev = torch.from_numpy(addr_B.view(np.int64)).to(device)
        p.rank_dev = torch.from_numpy(rank).to(device)
        p.alpha_dev = torch.from_numpy(alpha).to(device)
        return p


class PageAlloc:
    """The library's frame allocator of one page pool (host side)."""

    def __init__(self, n_frames: int):
        self._h = ctypes.c_void_p()
        _check(load().lora_page_alloc_create(int(n_frames), ctypes.byref(self._h)), "lora_page_alloc_create")
        self.n_frames = int(n_frames)

    def take(self, n: int) -> np.ndarray:
        out = np.zeros(max(int(n), 1), dtype=np.int32)
        _check(load().lora_page_alloc_take(self._h, int(n), out.ctypes.data), "lora_page_alloc_take")
        return out[: int(n)]

    def give(self, frames) -> None:
        f = np.ascontiguousarray(frames, dtype=np.int32)
        _check(load().lora_page_alloc_give(self._h, f.ctypes.data, int(f.size)), "lora_page_alloc_give")

    @property
    def free(self) -> int:
        return int(load().lora_page_alloc_free_count(self._h))

    def close(self):
        if self._h:
            load().lora_page_alloc_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def lora_pages_needed(nbytes: int, page_bytes: int) -> int:
    return int(load().lora_pages_needed(int(nbytes), int(page_bytes)))


@dataclass
class PagedPool:
    """Adapters held in fixed-size pages of one device pool, each matrix behind
    a device page table (int32 frames).  addr_A / addr_B hold the addresses of
    the page tables, so a Plan builds from this pool as from a DevicePool."""

    pages: object  # device uint8 [n_frames * page_bytes]
    page_bytes: int
    tables: object  # device int32: every page table, each 16-byte aligned
    table_host: np.ndarray
    frames_A: list  # host int32 frames of each adapter's A
    frames_B: list
    alloc: PageAlloc
    n_adapters: int
    dtype: str
    d_in: int
    d_out: int
    addr_A: np.ndarray
    addr_B: np.ndarray
    rank: np.ndarray
    alpha: np.ndarray
    addr_A_dev: object = None
    addr_B_dev: object = None
    rank_dev: object = None
    alpha_dev: object = None

    @property
    def max_rank(self) -> int:
        return int(self.rank.max()) if self.rank.size else 0

    @classmethod
    def from_problem(cls, prob, page_bytes: int = 16384, shuffle_seed: Optional[int] = 0, spare_frames: int = 0,
                     device="cuda", stream=None) -> "PagedPool":
        """Allocates frames for every adapter of `prob` and writes A_i and B_i
        into them with lora_pages_write.  shuffle_seed: frames are first taken
        and given back in a seeded random order, so each matrix lands in
        scattered frames (None: ascending frames)."""
        torch = _torch()
        es = prob.esize
        ranks = np.ascontiguousarray(prob.ranks, dtype=np.int32)
        nA = [lora_pages_needed(int(r) * prob.d_in * es, page_bytes) for r in ranks]
        nB = [lora_pages_needed(prob.d_out * int(r) * es, page_bytes) for r in ranks]
        if min(nA + nB, default=0) < 0:
            raise ValueError(f"page_bytes {page_bytes} is not a power of two in [64, 2^24]")
        n_frames = int(sum(nA) + sum(nB) + spare_frames)
        alloc = PageAlloc(max(n_frames, 1))
        if shuffle_seed is not None and n_frames > 0:
            all_frames = alloc.take(n_frames)
            alloc.give(np.random.default_rng(shuffle_seed).permutation(all_frames))
        frames_A = [alloc.take(n) for n in nA]
        frames_B = [alloc.take(n) for n in nB]
        # page tables, each starting on a 16-byte boundary
        offs_A, offs_B, parts, pos = [], [], [], 0
        for fa, fb in zip(frames_A, frames_B):
            for f, offs in ((fa, offs_A), (fb, offs_B)):
                offs.append(pos)
                pad = (-len(f)) % 4
                parts.append(np.concatenate([f, np.zeros(pad, dtype=np.int32)]))
                pos += len(f) + pad
        table_host = np.concatenate(parts) if parts else np.zeros(4, dtype=np.int32)
        tables = torch.from_numpy(table_host).to(device)
        base = tables.data_ptr()
        addr_A = np.array([base + 4 * o for o in offs_A], dtype=np.uint64)
        addr_B = np.array([base + 4 * o for o in offs_B], dtype=np.uint64)
        pages = torch.empty(max(n_frames, 1) * page_bytes, dtype=torch.uint8, device=device)
        dense = to_device(prob.pool, prob.dtype, device)
        sbase = dense.data_ptr()
        st = _stream_handle(stream)
        for i, r in enumerate(ranks):
            for off, nbytes, addr in ((int(prob.a_off[i]), int(r) * prob.d_in * es, addr_A[i]),
                                      (int(prob.b_off[i]), prob.d_out * int(r) * es, addr_B[i])):
                _check(load().lora_pages_write(st, pages.data_ptr(), page_bytes, int(addr), sbase + off * es,
                                               nbytes), "lora_pages_write")
        torch.cuda.synchronize()
        del dense
        alpha = np.ascontiguousarray(prob.alphas, dtype=np.float32)
        p = cls(pages=pages, page_bytes=int(page_bytes), tables=tables, table_host=table_host, frames_A=frames_A,
                frames_B=frames_B, alloc=alloc, n_adapters=prob.n_adapters, dtype=prob.dtype, d_in=prob.d_in,
                d_out=prob.d_out, addr_A=addr_A, addr_B=addr_B, rank=ranks, alpha=alpha)
        p.addr_A_dev = torch.from_numpy(addr_A.view(np.int64)).to(device)
        p.addr_B_dev = torch.from_numpy(addr_B.view(np.int64)).to(device)
        p.rank_dev = torch.from_numpy(ranks).to(device)
        p.alpha_dev = torch.from_numpy(alpha).to(device)
        return p


SEG_DESC = np.dtype([("A", "<u8"), ("B", "<u8"), ("start", "<i4"), ("len", "<i4"), ("rank", "<i4"),
                     ("adapter", "<i4"), ("scale", "<f4"), ("blk0", "<i4")])
BLK_DESC = np.dtype([("A", "<u8"), ("B", "<u8"), ("scale", "<f4"), ("rank", "<i4"), ("n", "<i4"), ("p0", "<i4"),
                     ("seg", "<i4"), ("reserved", "<i4", (7,)), ("rows", "<i4", (ROW_BLOCK,))])
CHUNK_DESC = np.dtype([("A", "<u8"), ("B", "<u8"), ("scale", "<f4"), ("rank", "<i4"), ("n", "<i4"),
                       ("p0", "<i4"), ("seg", "<i4"), ("first_blk", "<i4"), ("nblk", "<i4"),
                       ("reserved", "<i4", (5,)), ("rows", "<i4", (ROW_BLOCK * CHUNK_BLOCKS,))])
assert SEG_DESC.itemsize == 40 and BLK_DESC.itemsize == 128 and CHUNK_DESC.itemsize == 320


def plan_header(h: np.ndarray) -> dict:
    """Fields of a plan header held in `h` (uint8, at least 96 bytes)."""
    i32 = h[:32].view(np.int32)
    u64 = h[32:96].view(np.uint64)
    return {"magic": int(h[:4].view(np.uint32)[0]), "num_tokens": int(i32[1]), "num_sorted": int(i32[2]),
            "num_segments": int(i32[3]), "num_blocks": int(i32[4]), "max_rank": int(i32[5]),
            "max_len": int(i32[6]), "num_chunks": int(i32[7]), "seg_offset": int(u64[0]),
            "blk_offset": int(u64[1]), "perm_offset": int(u64[2]), "bytes_used": int(u64[3]),
            "chunk_offset": int(u64[4]), "segidx_offset": int(u64[5]), "soa_offset": int(u64[6])}


def plan_arrays(buf: np.ndarray, h: dict) -> dict:
    """Segment descriptors, block descriptors and perm of a plan held in `buf` (uint8)."""
    S, nb, Tp = h["num_segments"], h["num_blocks"], h["num_sorted"]
    so, bo, po = h["seg_offset"], h["blk_offset"], h["perm_offset"]
    seg = np.frombuffer(buf[so: so + SEG_DESC.itemsize * S].tobytes(), dtype=SEG_DESC)
    blk = np.frombuffer(buf[bo: bo + BLK_DESC.itemsize * nb].tobytes(), dtype=BLK_DESC)
    perm = buf[po: po + 4 * Tp].view(np.int32).copy()
    rest = buf[po + 4 * Tp: po + 4 * h["num_tokens"]].view(np.int32).copy()
    out = {"desc": seg, "blocks": blk, "perm": perm, "unadapted": rest}
    if "segidx_offset" in h:
        xo = h["segidx_offset"]
        out["segidx"] = buf[xo: xo + 4 * Tp].view(np.int32).copy()
    if "chunk_offset" in h:
        co = h["chunk_offset"]
        out["chunks"] = np.frombuffer(buf[co: co + CHUNK_DESC.itemsize * h["num_chunks"]].tobytes(), dtype=CHUNK_DESC)
    return out


class Plan:
    """A batch's segments (struct lora_segments): a pinned host buffer and a
    device buffer, each bound to a struct; build() fills the host one,
    upload() copies it to the device one (one copy).  `seg` is the address of
    the device struct, which the calls take."""

    def __init__(self, capacity: int, device="cuda"):
        torch = _torch()
        self.capacity = int(capacity)
        self.nbytes = lora_segments_bytes(self.capacity)
        self.host = torch.empty(self.nbytes, dtype=torch.uint8, pin_memory=True)
        self.dev = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        self.h = LoraSegments()
        self.d = LoraSegments()
        _check(lora_segments_bind(self.host.data_ptr(), self.capacity, ctypes.addressof(self.h)), "lora_segments_bind")
        _check(lora_segments_bind(self.dev.data_ptr(), self.capacity, ctypes.addressof(self.d)), "lora_segments_bind")

    @property
    def seg(self) -> int:
        return ctypes.addressof(self.d)

    def build(self, ids: np.ndarray, pool: DevicePool):
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        if ids.shape[0] > self.capacity:
            raise ValueError("batch larger than the segments' capacity")
        st = lora_build_segments(ids.shape[0], ids.ctypes.data, pool.n_adapters, pool.addr_A.ctypes.data,
                                 pool.addr_B.ctypes.data, pool.rank.ctypes.data, pool.alpha.ctypes.data,
                                 ctypes.addressof(self.h))
        _check(st, "lora_build_segments")
        return self

    def upload(self, stream=None):
        _check(lora_segments_upload(ctypes.addressof(self.h), ctypes.addressof(self.d), _stream_handle(stream)),
               "lora_segments_upload")
        return self

    def header(self) -> dict:
        return plan_header(self.host[:PLAN_HEADER_BYTES].numpy())

    def arrays(self) -> dict:
        """Host copies of the plan's arrays (for tests)."""
        return plan_arrays(self.host.numpy(), self.header())

    def segment_table(self) -> dict:
        """The host struct's segment table as numpy arrays (copies)."""
        return segment_table(self.h)


_NP_OF = {ctypes.c_int32: np.int32, ctypes.c_uint64: np.uint64, ctypes.c_float: np.float32}


def segment_table(h: LoraSegments) -> dict:
    """perm, seg_indptr, seg_adapter, seg_rank, seg_A, seg_B, seg_scale of a
    host-bound struct, as numpy copies."""
    S, Tp = h.num_segments, h.num_tokens

    def arr(ptr, ctype, n):
        if n == 0 or not ptr:
            return np.zeros(0, dtype=_NP_OF[ctype])
        return np.ctypeslib.as_array(ctypes.cast(ptr, ctypes.POINTER(ctype)), (n,)).copy()

    return {"perm": arr(h.perm, ctypes.c_int32, Tp), "seg_indptr": arr(h.seg_indptr, ctypes.c_int32, S + 1),
            "seg_adapter": arr(h.seg_adapter, ctypes.c_int32, S), "seg_rank": arr(h.seg_rank, ctypes.c_int32, S),
            "seg_A": arr(h.seg_A, ctypes.c_uint64, S), "seg_B": arr(h.seg_B, ctypes.c_uint64, S),
            "seg_scale": arr(h.seg_scale, ctypes.c_float, S)}


def sgmv_shrink(x, plan: Plan, v, dtype: str, stream=None):
    d_in = x.shape[1]
    _check(lora_sgmv_shrink(_stream_handle(stream), DTYPES[dtype], _ptr(x), x.stride(0), d_in,
                            plan.seg, _ptr(v), v.stride(0), None, 0),
           "lora_sgmv_shrink")


def sgmv_expand(v, plan: Plan, y, dtype: str, stream=None):
    _check(lora_sgmv_expand(_stream_handle(stream), DTYPES[dtype], _ptr(v), v.stride(0), plan.seg, _ptr(y),
                            y.stride(0), y.shape[1], None, 0),
           "lora_sgmv_expand")


def workspace(op: int, T: int, d_in: int, d_out: int, max_rank: int, device="cuda"):
    """A zero-filled device workspace of the size the library asks for (uint8
    tensor; lora_bgmv needs its control words zero before the first call)."""
    torch = _torch()
    n = lora_workspace_bytes(op, T, d_in, d_out, max_rank)
    return torch.zeros(max(n, 16), dtype=torch.uint8, device=device)


def workspace_clear(ws, stream=None):
    """lora_workspace_clear on a workspace tensor."""
    _check(load().lora_workspace_clear(_stream_handle(stream), _ptr(ws), ws.numel() * ws.element_size()),
           "lora_workspace_clear")


def workspace_status(ws) -> int:
    """The status word at the start of a BGMV workspace (synchronises)."""
    return int(ws[:4].view(_torch().int32).item())


def debug_wait_limit(polls: int):
    _check(load().lora_debug_wait_limit(int(polls)), "lora_debug_wait_limit")


def sgmv(x, plan: Plan, y, ws, dtype: str, stream=None):
    """y[perm] += scale (x[perm] A) B for the whole plan (shrink + expand)."""
    _check(lora_sgmv(_stream_handle(stream), DTYPES[dtype], _ptr(x), x.stride(0), x.shape[1], plan.seg, _ptr(y),
                     y.stride(0), y.shape[1], _ptr(ws), ws.numel() * ws.element_size()),
           "lora_sgmv")


def bgmv(x, ids_dev, pool: DevicePool, y, ws, dtype: str, max_rank: Optional[int] = None, stream=None):
    """Decode: y[t] += scale (x[t] A_ids[t]) B_ids[t] (shrink + expand)."""
    _check(lora_bgmv(_stream_handle(stream), DTYPES[dtype], x.shape[0], _ptr(x), x.stride(0), x.shape[1],
                     _ptr(ids_dev), _ptr(pool.addr_A_dev), _ptr(pool.addr_B_dev), _ptr(pool.rank_dev),
                     _ptr(pool.alpha_dev), pool.n_adapters, max_rank or pool.max_rank, _ptr(y), y.stride(0),
                     y.shape[1], _ptr(ws), ws.numel() * ws.element_size()),
           "lora_bgmv")


def sgmv_prepared(x, plan: Plan, y, ws, dtype: str, stream) -> Prepared:
    """lora_sgmv with its arguments converted once (see Prepared)."""
    return Prepared("lora_sgmv", (_stream_handle(stream), DTYPES[dtype], _ptr(x), x.stride(0), x.shape[1],
                                  plan.seg, _ptr(y), y.stride(0), y.shape[1],
                                  _ptr(ws), ws.numel() * ws.element_size()), keep=(x, plan, y, ws))


def bgmv_prepared(x, ids_dev, pool, y, ws, dtype: str, stream, max_rank: Optional[int] = None) -> Prepared:
    """lora_bgmv with its arguments converted once (see Prepared)."""
    return Prepared("lora_bgmv", (_stream_handle(stream), DTYPES[dtype], x.shape[0], _ptr(x), x.stride(0),
                                  x.shape[1], _ptr(ids_dev), _ptr(pool.addr_A_dev), _ptr(pool.addr_B_dev),
                                  _ptr(pool.rank_dev), _ptr(pool.alpha_dev), pool.n_adapters,
                                  max_rank or pool.max_rank, _ptr(y), y.stride(0), y.shape[1], _ptr(ws),
                                  ws.numel() * ws.element_size()), keep=(x, ids_dev, pool, y, ws))


def sgmv_paged_prepared(x, plan: Plan, pool: "PagedPool", y, ws, dtype: str, stream) -> Prepared:
    return Prepared("lora_sgmv_paged", (_stream_handle(stream), DTYPES[dtype], _ptr(x), x.stride(0), x.shape[1],
                                        plan.seg, _ptr(pool.pages),
                                        pool.page_bytes, _ptr(y), y.stride(0), y.shape[1], _ptr(ws),
                                        ws.numel() * ws.element_size()), keep=(x, plan, pool, y, ws))


def bgmv_paged_prepared(x, ids_dev, pool: "PagedPool", y, ws, dtype: str, stream,
                        max_rank: Optional[int] = None) -> Prepared:
    return Prepared("lora_bgmv_paged", (_stream_handle(stream), DTYPES[dtype], x.shape[0], _ptr(x), x.stride(0),
                                        x.shape[1], _ptr(ids_dev), _ptr(pool.addr_A_dev), _ptr(pool.addr_B_dev),
                                        _ptr(pool.rank_dev), _ptr(pool.alpha_dev), pool.n_adapters,
                                        max_rank or pool.max_rank, _ptr(pool.pages), pool.page_bytes, _ptr(y),
                                        y.stride(0), y.shape[1], _ptr(ws), ws.numel() * ws.element_size()),
                    keep=(x, ids_dev, pool, y, ws))


def fused_prepared(x, W0, plan: Plan, y, ws, dtype: str, stream) -> Prepared:
    return Prepared("lora_fused_linear", (_stream_handle(stream), DTYPES[dtype], _ptr(x), x.stride(0), x.shape[1],
                                          _ptr(W0), W0.shape[0], plan.seg,
                                          _ptr(y), y.stride(0), _ptr(ws), ws.numel() * ws.element_size()),
                    keep=(x, W0, plan, y, ws))


def fused_e4m3_prepared(x, W0, w0_scale: float, plan: Plan, y, ws, stream) -> Prepared:
    """W0: uint8 E4M3 codes [d_out, d_in] standing for w0_scale * code."""
    return Prepared("lora_fused_linear_e4m3", (_stream_handle(stream), _ptr(x), x.stride(0), x.shape[1], _ptr(W0),
                                               float(w0_scale), W0.shape[0], plan.seg, _ptr(y), y.stride(0), _ptr(ws),
                                               ws.numel() * ws.element_size()),
                    keep=(x, W0, plan, y, ws))


def sgmv_grouped_prepared(projs, ws, dtype: str, stream, keep=()) -> Prepared:
    return Prepared("lora_sgmv_grouped", (_stream_handle(stream), DTYPES[dtype], ctypes.cast(projs, _vp).value,
                                          len(projs), _ptr(ws), ws.numel() * ws.element_size()),
                    keep=(projs, ws, *keep))


def bgmv_grouped_prepared(T: int, ids_dev, n_adapters: int, projs, ws, dtype: str, stream, keep=()) -> Prepared:
    return Prepared("lora_bgmv_grouped", (_stream_handle(stream), DTYPES[dtype], T, _ptr(ids_dev), n_adapters,
                                          ctypes.cast(projs, _vp).value, len(projs), _ptr(ws),
                                          ws.numel() * ws.element_size()), keep=(ids_dev, projs, ws, *keep))


def sgmv_paged(x, plan: Plan, pool: PagedPool, y, ws, dtype: str, stream=None):
    """lora_sgmv over paged adapters (plan built from the PagedPool)."""
    _check(load().lora_sgmv_paged(_stream_handle(stream), DTYPES[dtype], _ptr(x), x.stride(0), x.shape[1],
                                  plan.seg, _ptr(pool.pages), pool.page_bytes,
                                  _ptr(y), y.stride(0), y.shape[1], _ptr(ws), ws.numel() * ws.element_size()),
           "lora_sgmv_paged")


def bgmv_paged(x, ids_dev, pool: PagedPool, y, ws, dtype: str, max_rank: Optional[int] = None, stream=None):
    """lora_bgmv over paged adapters."""
    _check(load().lora_bgmv_paged(_stream_handle(stream), DTYPES[dtype], x.shape[0], _ptr(x), x.stride(0),
                                  x.shape[1], _ptr(ids_dev), _ptr(pool.addr_A_dev), _ptr(pool.addr_B_dev),
                                  _ptr(pool.rank_dev), _ptr(pool.alpha_dev), pool.n_adapters,
                                  max_rank or pool.max_rank, _ptr(pool.pages), pool.page_bytes, _ptr(y), y.stride(0),
                                  y.shape[1], _ptr(ws), ws.numel() * ws.element_size()),
           "lora_bgmv_paged")


def sgmv_proj_array(xs, plans, ys):
    """Host array of struct lora_sgmv_proj for projections (xs[p], plans[p], ys[p])."""
    arr = (LoraSgmvProj * len(xs))()
    for p, (x, plan, y) in enumerate(zip(xs, plans, ys)):
        arr[p] = LoraSgmvProj(_ptr(x), _ptr(y), plan.seg, x.stride(0), y.stride(0),
                              x.shape[1], y.shape[1])
    return arr


def sgmv_grouped_workspace(plans_or_projs, xs=None, ys=None, device="cuda"):
    """A device workspace for lora_sgmv_grouped (uint8 tensor)."""
    torch = _torch()
    projs = plans_or_projs if xs is None else sgmv_proj_array(xs, plans_or_projs, ys)
    n = int(load().lora_sgmv_grouped_workspace_bytes(projs, len(projs)))
    if n == 0:
        raise LoraError(-1, "lora_sgmv_grouped_workspace_bytes", "invalid projections")
    return torch.empty(n, dtype=torch.uint8, device=device)


def sgmv_grouped(xs, plans, ys, ws, dtype: str, stream=None, projs=None):
    """Prefill correction of several projections in one shrink and one expand
    launch: projection p applies plans[p] (built from the batch's ids with its
    own adapter tables) to xs[p] and accumulates into ys[p]."""
    projs = projs if projs is not None else sgmv_proj_array(xs, plans, ys)
    _check(load().lora_sgmv_grouped(_stream_handle(stream), DTYPES[dtype], projs, len(projs), _ptr(ws),
                                    ws.numel() * ws.element_size()), "lora_sgmv_grouped")


def proj_array(xs, pools, ys, max_ranks=None):
    """Host array of struct lora_proj for projections (xs[p], pools[p], ys[p])."""
    n = len(xs)
    arr = (LoraProj * n)()
    for p in range(n):
        x, pool, y = xs[p], pools[p], ys[p]
        arr[p] = LoraProj(_ptr(x), _ptr(y), _ptr(pool.addr_A_dev), _ptr(pool.addr_B_dev), _ptr(pool.rank_dev),
                          _ptr(pool.alpha_dev), x.stride(0), y.stride(0), x.shape[1], y.shape[1],
                          int(max_ranks[p]) if max_ranks is not None else max(pool.max_rank, 1), 0)
    return arr


def bgmv_grouped_workspace(T: int, projs, device="cuda"):
    torch = _torch()
    nbytes = lora_bgmv_grouped_workspace_bytes(T, ctypes.cast(projs, _vp), len(projs))
    if nbytes == 0 and T > 0:
        raise ValueError("invalid projections for a grouped workspace")
    # zero-filled: the status word at its start must begin at zero
    return torch.zeros(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def bgmv_grouped(xs, ids_dev, pools, ys, ws, dtype: str, max_ranks=None, stream=None, projs=None):
    """Decode for several projections in one shrink and one expand launch:
    ys[p][t] += scale (xs[p][t] A_{ids[t],p}) B_{ids[t],p}.  All pools share the
    adapter numbering of ids_dev."""
    n_adapters = pools[0].n_adapters
    if any(p.n_adapters != n_adapters for p in pools):
        raise ValueError("every projection's pool must number the same adapters as ids_dev")
    if projs is None:
        projs = proj_array(xs, pools, ys, max_ranks)
    T = xs[0].shape[0]
    _check(lora_bgmv_grouped(_stream_handle(stream), DTYPES[dtype], T, _ptr(ids_dev), n_adapters,
                             ctypes.cast(projs, _vp), len(projs), _ptr(ws), ws.numel() * ws.element_size()),
           "lora_bgmv_grouped")


def bgmv_shrink(x, ids_dev, pool: DevicePool, v, dtype: str, max_rank: Optional[int] = None, stream=None):
    _check(lora_bgmv_shrink(_stream_handle(stream), DTYPES[dtype], x.shape[0], _ptr(x), x.stride(0), x.shape[1],
                            _ptr(ids_dev), _ptr(pool.addr_A_dev), _ptr(pool.rank_dev), pool.n_adapters,
                            max_rank or pool.max_rank, _ptr(v), v.stride(0), None, 0),
           "lora_bgmv_shrink")


def bgmv_expand(v, ids_dev, pool: DevicePool, y, dtype: str, max_rank: Optional[int] = None, stream=None):
    _check(lora_bgmv_expand(_stream_handle(stream), DTYPES[dtype], y.shape[0], _ptr(v), v.stride(0), _ptr(ids_dev),
                            _ptr(pool.addr_B_dev), _ptr(pool.rank_dev), _ptr(pool.alpha_dev), pool.n_adapters,
                            max_rank or pool.max_rank, _ptr(y), y.stride(0), y.shape[1], None, 0),
           "lora_bgmv_expand")


def fused_linear(x, W0, plan: Plan, y, ws, dtype: str = "bf16", stream=None):
    _check(lora_fused_linear(_stream_handle(stream), DTYPES[dtype], _ptr(x), x.stride(0), x.shape[1], _ptr(W0),
                             W0.shape[0], plan.seg, _ptr(y), y.stride(0),
                             _ptr(ws), ws.numel() * ws.element_size()),
           "lora_fused_linear")


def fused_linear_e4m3(x, W0, w0_scale: float, plan: Plan, y, ws, stream=None):
    """The fused layer over an FP8 base: W0 holds uint8 E4M3 codes [d_out, d_in]
    standing for w0_scale * code; x, y and the adapters are bf16."""
    _check(lora_fused_linear_e4m3(_stream_handle(stream), _ptr(x), x.stride(0), x.shape[1], _ptr(W0),
                                  float(w0_scale), W0.shape[0], plan.seg, _ptr(y), y.stride(0),
                                  _ptr(ws), ws.numel() * ws.element_size()),
           "lora_fused_linear_e4m3")


def v_pitch(max_rank: int) -> int:
    """Row pitch (fp32 elements) for v: max rank rounded up to a multiple of 4."""
    return max(4, (int(max_rank) + 3) // 4 * 4)
