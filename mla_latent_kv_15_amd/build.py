"""Build libmla.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""

from __future__ import annotations

import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla.so")
ARCH = os.environ.get("MLA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["mla_host.cpp", "mla_kernels.hip", "mla_decode_fp8.hip", "mla_prefill.hip"]

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Kernels whose matrix accumulators are named as fixed AGPRs in inline asm
# (the compiler does not see them as values): the build fails unless the
# compiler keeps its own registers out of the AGPR file, i.e. no spills, no
# scratch, fewer than 256 VGPRs (a full VGPR file is where it would start
# parking values in AGPRs), and all 256 AGPRs allocated.
FIXED_AGPR_KERNELS = ("decode_h128_kernel",)


def resource_usage(remarks: str) -> dict:
    """{kernel symbol: {key: value}} from -Rpass-analysis=kernel-resource-usage."""
    out, cur = {}, None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][^:]*):\s+(\S+) \[-Rpass-analysis", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return out


def check_fixed_agpr_kernels(usage: dict) -> None:
    found = [k for k in usage if any(f in k for f in FIXED_AGPR_KERNELS)]
    if not found:
        raise RuntimeError("no resource usage reported for the fixed-AGPR kernels")
    for k in found:
        u = usage[k]
        ok = (u.get("VGPRs Spill") == "0" and u.get("ScratchSize [bytes/lane]") == "0"
              and int(u.get("VGPRs", 256)) < 256 and u.get("AGPRs") == "256")
        if not ok:
            raise RuntimeError(f"{k}: the compiler's registers reach the fixed accumulators: {u}")


def build(verbose: bool = False, extra: list | None = None) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *HIPFLAGS, "-Rpass-analysis=kernel-resource-usage", *(extra or []), *srcs,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd=CSRC, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise subprocess.CalledProcessError(r.returncode, cmd)
    check_fixed_agpr_kernels(resource_usage(r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
