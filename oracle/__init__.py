"""ctypes wrapper of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the product path may not.  The
oracle shares no code with the GPU library.

Functions and what they follow:

* ``lora_forward`` -- per-token layer output x W0 (or the stored base output)
  plus (alpha/r) (x A) B in fp64 ("Multi-LoRA Serving in Production ..."
  (llms.blog), section "Mathematical Formulation and the Batching Challenge";
  per-token adapter a(t) from "Multi-LoRA serving: the single translator ..."
  (blog.lo0.es), section "SGMV: the kernel that holds it all up").
* ``segments`` -- brute-force grouping of tokens by adapter id into contiguous
  segments ("Multi-LoRA Serving in Production ...", section "Punica and
  Segmented Gather Matrix-Vector Multiplication (SGMV)"), ascending id, stable.
* ``e4m3_decode`` -- the value of each 8-bit E4M3 code, exactly, from the
  format's definition (OCP 8-bit floating point specification, E4M3 encoding);
  ``lora_forward`` uses it for an FP8 base W0 = w0_scale * codes ("Multi-LoRA
  serving: the single translator ...", section "Combined pattern with
  quantisation and disaggregated serving": BF16 adapters over an FP8 base).
* ``adapter_numel`` / ``adapter_bytes`` -- r (d_in + d_out) parameters
  ("Multi-LoRA Serving: Many Adapters on One GPU" (gpusmith.com), section "LoRA
  recap and why adapters are small"; bytes per matrix from "Multi-LoRA serving:
  the single translator ...", section "The maths that matters").
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_BUILD = os.path.join(_HERE, "_build")
_LOCK = threading.Lock()
_LIBS: dict = {}

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def lib_path(mutant: int = 0) -> str:
    name = "liboracle.so" if mutant == 0 else f"liboracle_mutant{mutant}.so"
    return os.path.join(_BUILD, name)


def build(mutant: int = 0, force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, fp64, no fast-math, OpenMP over tokens)."""
    out = lib_path(mutant)
    src = os.path.join(_HERE, "oracle.c")
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    os.makedirs(_BUILD, exist_ok=True)
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           f"-DORACLE_MUTANT={int(mutant)}", os.path.join(_HERE, "oracle.c"), "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _load(mutant: int = 0):
    with _LOCK:
        if mutant in _LIBS:
            return _LIBS[mutant]
        path = lib_path(mutant)
        if not os.path.exists(path):
            build(mutant)
        lib = ctypes.CDLL(path)
        lib.oracle_mutant_id.restype = ctypes.c_int
        lib.oracle_adapter_numel.restype = _i64
        lib.oracle_adapter_numel.argtypes = [_i32, _i32, _i32]
        lib.oracle_adapter_bytes.restype = _i64
        lib.oracle_adapter_bytes.argtypes = [_i32, _i32, _i32, _i32]
        lib.oracle_segments.restype = _i32
        lib.oracle_segments.argtypes = [_i32, _vp, _i32, _vp, _vp, _vp]
        lib.oracle_lora_forward.restype = ctypes.c_int
        lib.oracle_lora_forward.argtypes = [
            _i32, _i32, _i32, _i32, _vp, _i64, _vp, _i32, _vp, _vp, _vp, _vp, _vp,
            _vp, _i64, _vp, _i32, ctypes.c_double, _vp, _i64, _vp, _i32]
        lib.oracle_e4m3_decode.restype = None
        lib.oracle_e4m3_decode.argtypes = [_vp, _i64, _vp]
        assert lib.oracle_mutant_id() == mutant
        _LIBS[mutant] = lib
        return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def adapter_numel(r: int, d_in: int, d_out: int, mutant: int = 0) -> int:
    return int(_load(mutant).oracle_adapter_numel(r, d_in, d_out))


def adapter_bytes(r: int, d_in: int, d_out: int, bytes_per_param: int = 2, mutant: int = 0) -> int:
    return int(_load(mutant).oracle_adapter_bytes(r, d_in, d_out, bytes_per_param))


def segments(ids, n_adapters: int, mutant: int = 0):
    """Returns (perm int32[T'], seg_indptr int32[S+1], seg_adapter int32[S])."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T = int(ids.shape[0])
    perm = np.zeros(max(T, 1), dtype=np.int32)
    indptr = np.zeros(max(T, 1) + 1, dtype=np.int32)
    adapter = np.zeros(max(T, 1), dtype=np.int32)
    S = _load(mutant).oracle_segments(T, _ptr(ids), n_adapters, _ptr(perm), _ptr(indptr), _ptr(adapter))
    if S < 0:
        raise ValueError("adapter id out of range")
    n = int(indptr[S])
    return perm[:n].copy(), indptr[: S + 1].copy(), adapter[:S].copy()


def e4m3_decode(codes, mutant: int = 0) -> np.ndarray:
    """float64 values of uint8 E4M3 codes (NaN for the two NaN codes)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _load(mutant).oracle_e4m3_decode(_ptr(c), int(c.size), _ptr(out))
    return out


def lora_forward(prob, *, nthreads: int = 1, want_v: bool = False, fused: bool = None,
                 ids=None, alphas=None, pool=None, mutant: int = 0):
    """fp64 layer output for a ``lora_workloads.LoraProblem``.

    fused=True uses x W0 as the base: W0 = prob.w0_scale * prob.W0_e4m3 when
    the problem holds E4M3 codes, else prob.W0 (one of them must exist);
    otherwise the base is prob.y_in (zeros if None).  ``ids``, ``alphas`` and ``pool`` override the
    problem's arrays (for invariance tests).  Returns (y, v) with v None unless
    want_v; v rows of tokens without an adapter are zero.
    """
    lib = _load(mutant)
    if fused is None:
        fused = bool(prob.meta.get("fused", False))
    is_bf16 = 1 if prob.dtype == "bf16" else 0
    ids = np.ascontiguousarray(prob.ids if ids is None else ids, dtype=np.int32)
    alphas = np.ascontiguousarray(prob.alphas if alphas is None else alphas, dtype=np.float32)
    pool = np.ascontiguousarray(prob.pool if pool is None else pool)
    ranks = np.ascontiguousarray(prob.ranks, dtype=np.int32)
    x = np.ascontiguousarray(prob.x)
    y_in = None if (fused or prob.y_in is None) else np.ascontiguousarray(prob.y_in)
    w0_codes = getattr(prob, "W0_e4m3", None) if fused else None
    if w0_codes is not None:
        W0 = np.ascontiguousarray(w0_codes, dtype=np.uint8)
    else:
        W0 = np.ascontiguousarray(prob.W0) if (fused and prob.W0 is not None) else None
    if fused and W0 is None:
        raise ValueError("fused oracle run needs W0")
    w0_scale = float(getattr(prob, "w0_scale", 1.0))
    T = prob.T
    y = np.zeros((T, prob.d_out), dtype=np.float64)
    ldv = max(prob.max_rank, 1)
    v = np.zeros((T, ldv), dtype=np.float64) if want_v else None
    rc = lib.oracle_lora_forward(
        T, prob.d_in, prob.d_out, is_bf16, _ptr(x), prob.d_in, _ptr(ids), prob.n_adapters,
        _ptr(pool), _ptr(np.ascontiguousarray(prob.a_off, dtype=np.int64)),
        _ptr(np.ascontiguousarray(prob.b_off, dtype=np.int64)), _ptr(ranks), _ptr(alphas),
        _ptr(y_in), prob.d_out, _ptr(W0), 1 if w0_codes is not None else 0, w0_scale, _ptr(v), ldv, _ptr(y),
        int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the problem (bad id or rank)")
    return y, v
