"""The host paths of the C ABI (plan parsing and validation, size queries,
argument checks, the offline planner) under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

Builds the library with host-code sanitizers (device code as usual) and
runs tests/test_abi_host.py and tests/test_planner.py against it in a child
process, with clang's ASan runtime preloaded (Python itself is not
instrumented, so leak checking is off).  Any sanitizer report aborts the
child and fails this test.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from loop_aware_quantized_amd import build as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.timeout(600)
def test_host_paths_clean_under_asan_and_ubsan():
    rt = _asan_runtime()
    if rt is None or shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc or the clang ASan runtime is not available")
    lib = b.build(sanitize=True)
    env = dict(os.environ, LOOPKV_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          "tests/test_abi_host.py", "tests/test_planner.py"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=500)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
