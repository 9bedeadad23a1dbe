"""Builds libdust.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdust.so")
SOURCES = [os.path.join(CSRC, "dust_kernels.hip"), os.path.join(CSRC, "dust_host.cpp")]
COMMON_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17",
    # keep the compiler from emitting packed fp32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
# -z defs: a symbol the library references but does not define fails the link
HIPCC_FLAGS = COMMON_FLAGS + ["-fPIC", "-shared", "-Wl,-z,defs"]


def build_library(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = f"{LIB}.{os.getpid()}.tmp"  # concurrent builds each write their own
    cmd = [hipcc, *HIPCC_FLAGS, "-o", tmp, *SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
