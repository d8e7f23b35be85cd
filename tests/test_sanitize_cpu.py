"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* oracle/oracle.c with the driver tests/c/oracle_sanitize.c, built with gcc
  (-fsanitize=address,undefined, no recovery);
* the library's host files (csrc/abi.cpp, csrc/residency.cpp) built with the
  sanitizers on their host code only, linked with the library's other objects
  as built (device kernels and their launchers, not instrumented) and the
  driver tests/c/host_sanitize.c, which exercises segment building, size
  queries, the page-frame allocator, the residency cache in its
  placement-only mode and the argument checks of the GPU calls (no GPU work).

Either driver aborts at the first sanitizer report; the test also fails on
any report text in its output.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "segmented_gather_gemm_lora_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    out = res.stdout + res.stderr
    assert res.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({res.returncode}):\n{out[-4000:]}"
    return out


def _no_report(out):
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer"):
        assert marker not in out, out[-4000:]


def test_oracle_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_sanitize")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", os.path.join(ROOT, "tests", "c", "oracle_sanitize.c"),
          os.path.join(ROOT, "oracle", "oracle.c"), "-o", exe, "-lm"])
    out = _run([exe], env=ENV, timeout=300)
    _no_report(out)
    assert "oracle_sanitize: ok" in out


def test_host_library_under_sanitizers():
    from segmented_gather_gemm_lora_amd import build as bld

    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    clang = "/opt/rocm/llvm/bin/clang++"
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm toolchain not found")
    # the device-code objects as the library build makes them
    objs = [os.path.join(bld.OBJ_DIR, os.path.splitext(s)[0] + ".o") for s in bld.SOURCES
            if s not in ("abi.cpp", "residency.cpp")]
    if not all(os.path.exists(o) for o in objs):
        bld.build(verbose=False)
    os.makedirs(OUT, exist_ok=True)
    san_objs = []
    for src in ("abi.cpp", "residency.cpp"):
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        # sanitizers on the host pass only (each -fsanitize after -Xarch_host)
        _run([hipcc, *bld.HIPCC_FLAGS, "-O1", "-g", "-fno-omit-frame-pointer",
              "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=all", "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
        san_objs.append(obj)
    drv = os.path.join(OUT, "host_sanitize.o")
    _run([clang, "-x", "c", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          f"-I{os.path.join(ROOT, 'include')}", "-c", os.path.join(ROOT, "tests", "c", "host_sanitize.c"), "-o", drv])
    exe = os.path.join(OUT, "host_sanitize")
    _run([clang, "-fsanitize=address,undefined", drv, *san_objs, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    out = _run([exe], env=ENV, timeout=300)
    _no_report(out)
    assert "host_sanitize: ok" in out
