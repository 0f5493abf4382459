"""The build's guard for the kernel whose accumulators are fixed AGPRs named in
inline asm: it reads the compiler's resource-usage remarks and rejects a
build in which the compiler's own registers could reach those AGPRs."""

import importlib

import pytest

build = importlib.import_module("mla_latent_kv_15_amd.build")

K = "_ZN3mla12_GLOBAL__N_118decode_h128_kernelILi1EEEvNS0_12DecodeParamsEPKi"


def remarks(vgprs=221, agprs=256, spill=0, scratch=0):
    r = "mla_kernels.hip:917:1: remark: {} [-Rpass-analysis=kernel-resource-usage]\n"
    return "".join(r.format(x) for x in (
        f"Function Name: {K}", "    TotalSGPRs: 102", f"    VGPRs: {vgprs}", f"    AGPRs: {agprs}",
        f"    ScratchSize [bytes/lane]: {scratch}", "    Occupancy [waves/SIMD]: 1",
        f"    VGPRs Spill: {spill}", "    LDS Size [bytes/block]: 163840"))


def test_parses_the_remarks():
    u = build.resource_usage(remarks())
    assert u[K]["VGPRs"] == "221" and u[K]["AGPRs"] == "256" and u[K]["VGPRs Spill"] == "0"
    build.check_fixed_agpr_kernels(u)


@pytest.mark.parametrize("kw", [dict(spill=4), dict(scratch=16), dict(vgprs=256), dict(agprs=128)])
def test_rejects_a_build_that_reaches_the_fixed_agprs(kw):
    with pytest.raises(RuntimeError):
        build.check_fixed_agpr_kernels(build.resource_usage(remarks(**kw)))


def test_rejects_missing_remarks():
    with pytest.raises(RuntimeError):
        build.check_fixed_agpr_kernels(build.resource_usage(""))
