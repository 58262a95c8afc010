"""Host-only C++ of the library under AddressSanitizer + UndefinedBehaviorSanitizer.

Two drivers under ``tests/native/`` are built with g++ together with the
library's host translation units and run; every out-of-bounds access, use
after free, leak (where the HIP runtime is not linked), signed overflow or
misaligned access in those files fails the run.  CPU only, nothing touches a
device:

* ``host_abi_check.cpp`` with ``layout.cpp`` (block layout, ceil-division
  shard size, error reporting) and ``ops.cpp`` (validation and argument
  marshalling of the kernel-level entry points); the kernel launchers are
  recorders.
* ``runtime_host_check.cpp`` with ``layout.cpp`` and ``runtime.cpp`` (context,
  pinned shards, chunked staging, two-slot schedule, tracing, fail-closed
  errors) against an in-order fake of the HIP runtime in which device memory
  is host memory; the reconstruction launcher copies, the compute launchers
  check that the slot they read holds the block's bf16 weights bit-exactly.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "layerwise_weight_streaming_dit_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _toolchain_missing():
    if shutil.which("g++") is None:
        return "g++ not found"
    if not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        return "HIP headers not found"
    if not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        return "libamdhip64 not found"
    return None


@pytest.mark.skipif(_toolchain_missing() is not None, reason=str(_toolchain_missing()))
def test_host_abi_under_sanitizers(tmp_path):
    exe = tmp_path / "host_abi_check"
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include", f"-I{CSRC}",
           os.path.join(CSRC, "layout.cpp"), os.path.join(CSRC, "ops.cpp"),
           os.path.join(ROOT, "tests", "native", "host_abi_check.cpp"),
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    # leak checking is off: the HIP runtime library keeps process-lifetime
    # allocations of its own; everything else the sanitizers check stays on
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "host ABI checks passed" in r.stdout


@pytest.mark.skipif(_toolchain_missing() is not None, reason=str(_toolchain_missing()))
def test_sanitizer_flags_catch_a_planted_overflow(tmp_path):
    """The same flags do catch a heap overflow here (the check above is live)."""
    src = tmp_path / "overflow.cpp"
    src.write_text("#include <stdlib.h>\nint main(int argc, char**) {\n"
                   "  int* p = static_cast<int*>(malloc(4 * sizeof(int)));\n"
                   "  p[argc + 3] = 1;  // one past the end\n  int v = p[0];\n  free(p);\n  return v & 0;\n}\n")
    exe = tmp_path / "overflow"
    r = subprocess.run(["g++", "-g", "-O0", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        str(src), "-o", str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr


@pytest.mark.skipif(_toolchain_missing() is not None, reason=str(_toolchain_missing()))
def test_runtime_host_logic_under_sanitizers(tmp_path):
    """Shards, chunking, slot alternation across forwards, re-pointing,
    validation and fail-closed errors of runtime.cpp, with a fake HIP runtime."""
    exe = tmp_path / "runtime_host_check"
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include", f"-I{CSRC}",
           os.path.join(CSRC, "layout.cpp"), os.path.join(CSRC, "runtime.cpp"),
           os.path.join(ROOT, "tests", "native", "runtime_host_check.cpp"), "-lpthread", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    # no HIP runtime is linked: leak checking stays on
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "runtime host checks passed" in r.stdout
