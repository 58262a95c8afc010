"""Host-only C++ of the C ABI under AddressSanitizer + UndefinedBehaviorSanitizer.

Builds ``tests/native/host_abi_check.cpp`` together with the library's
host-only translation units (``layout.cpp``: block layout, ceil-division shard
size, error reporting; ``ops.cpp``: validation and argument marshalling of the
kernel-level entry points) with g++ and runs it.  The kernel launchers are
replaced by recorders in the driver, so nothing touches a device; every
out-of-bounds access, use after free, signed overflow or misaligned access in
those files fails the run.  CPU only.
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
