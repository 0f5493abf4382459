"""Build libmla.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla.so")
ARCH = os.environ.get("MLA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["mla_host.cpp", "mla_kernels.hip"]

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, extra: list | None = None) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *HIPFLAGS, *(extra or []), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=CSRC)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
