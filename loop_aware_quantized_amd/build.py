"""Build step of the HIP library: compiles csrc/*.hip for gfx950 into
loop_aware_quantized_amd/libloopkv.so (in-tree, so it travels with the
source tree).  Run as ``python -m loop_aware_quantized_amd.build``.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libloopkv.so")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "--offload-arch=gfx950",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the codec's fp32 division must be IEEE round-to-nearest
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libloopkv.so)")


# host-code sanitizers (the device code is built as usual): a library for
# running the CPU tests of the host paths under AddressSanitizer and
# UndefinedBehaviorSanitizer, loaded with the clang ASan runtime preloaded
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-shared-libasan"]
SANITIZED_LIB = os.path.join(PKG, "libloopkv_hostsan.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every HIP source into LIB (or, with sanitize, into
    SANITIZED_LIB with host sanitizers); always recompiles."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources under " + CSRC)
    target = SANITIZED_LIB if sanitize else LIB
    tmp = target + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(SANITIZE_FLAGS if sanitize else []), "-I", INCLUDE, "-I", CSRC, *srcs,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libloopkv.so")
    warn = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if warn and verbose:
        sys.stderr.write(warn + "\n")
    os.replace(tmp, target)
    return target


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize-host" in sys.argv[1:]))
