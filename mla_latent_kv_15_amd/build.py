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


# The two decode kernels of the automatic choice wait on their own tile loads
# with hand-counted s_waitcnt vmcnt(N).  A register spill adds scratch loads
# and stores to that counter: the counted waits stay correct (ops issued after
# a tile's loads only make vmcnt(N) wait for more) but then stall on scratch
# traffic inside the tile loop.  The build fails unless the compiler reports
# no VGPR spill and no scratch for them.  The balanced-partition instances of
# decode_ws_kernel (template argument BAL = true) carry their piece loop's
# values across each piece and are allowed a few spill slots, reloaded at
# piece boundaries (BALANCED_MAX_VGPR_SPILLS; the fp32-partial instance
# spills 4, the bf16 one none).
COUNTED_WAIT_KERNELS = ("decode_ws_kernel", "decode_f8q_kernel")
BALANCED_MAX_VGPR_SPILLS = 8


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


def check_counted_wait_kernels(usage: dict) -> None:
    for name in COUNTED_WAIT_KERNELS:
        found = [k for k in usage if name in k]
        if not found:
            raise RuntimeError(f"no resource usage reported for {name}")
        for k in found:
            u = usage[k]
            if "ELb1EE" in k:  # decode_ws_kernel<FP8, PART_DT, BAL = true>
                if int(u.get("VGPRs Spill", "0")) > BALANCED_MAX_VGPR_SPILLS:
                    raise RuntimeError(f"{k}: more spills than the balanced decode allows: {u}")
                continue
            if u.get("VGPRs Spill") != "0" or u.get("ScratchSize [bytes/lane]") != "0":
                raise RuntimeError(f"{k}: spills or scratch in a decode kernel with counted waits: {u}")


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
    check_counted_wait_kernels(resource_usage(r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
