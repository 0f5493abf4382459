"""The build's guard for the decode kernels of the automatic choice, whose
waits on their own tile loads are counted by hand: it reads the compiler's
resource-usage remarks and rejects a build in which one of them spills
registers or uses scratch (scratch traffic inside the tile loop would stall
those waits)."""

import importlib

import pytest

build = importlib.import_module("mla_latent_kv_15_amd.build")

NAMES = {
    "decode_ws_kernel": "_ZN3mla12_GLOBAL__N_116decode_ws_kernelILb0ELi1ELb0EEEvNS_12DecodeParamsEPKi",
    "decode_f8q_kernel": "_ZN3mla12_GLOBAL__N_117decode_f8q_kernelILi1EEEvNS_12DecodeParamsEPKi",
}


def remarks(spill=0, scratch=0, skip=None):
    r = "mla_kernels.hip:100:1: remark: {} [-Rpass-analysis=kernel-resource-usage]\n"
    out = []
    for short, k in NAMES.items():
        if short == skip:
            continue
        out += [f"Function Name: {k}", "    TotalSGPRs: 102", "    VGPRs: 128", "    AGPRs: 128",
                f"    ScratchSize [bytes/lane]: {scratch}", "    Occupancy [waves/SIMD]: 2",
                f"    VGPRs Spill: {spill}", "    LDS Size [bytes/block]: 157184"]
    return "".join(r.format(x) for x in out)


def test_parses_the_remarks():
    u = build.resource_usage(remarks())
    k = NAMES["decode_f8q_kernel"]
    assert u[k]["VGPRs"] == "128" and u[k]["AGPRs"] == "128" and u[k]["VGPRs Spill"] == "0"
    build.check_counted_wait_kernels(u)


@pytest.mark.parametrize("kw", [dict(spill=4), dict(scratch=16)])
def test_rejects_a_build_with_spills(kw):
    with pytest.raises(RuntimeError):
        build.check_counted_wait_kernels(build.resource_usage(remarks(**kw)))


@pytest.mark.parametrize("skip", sorted(NAMES))
def test_rejects_missing_remarks(skip):
    with pytest.raises(RuntimeError):
        build.check_counted_wait_kernels(build.resource_usage(remarks(skip=skip)))


BALANCED = "_ZN3mla12_GLOBAL__N_116decode_ws_kernelILb0ELi1ELb1EEEvNS_12DecodeParamsEPKi"


def _with_balanced(spill):
    r = "mla_kernels.hip:100:1: remark: {} [-Rpass-analysis=kernel-resource-usage]\n"
    extra = [f"Function Name: {BALANCED}", "    VGPRs: 128", "    ScratchSize [bytes/lane]: 20",
             f"    VGPRs Spill: {spill}"]
    return remarks() + "".join(r.format(x) for x in extra)


def test_balanced_instances_may_spill_a_little():
    """the balanced-partition instances carry their piece loop's values and
    may spill up to the stated bound, not beyond"""
    build.check_counted_wait_kernels(build.resource_usage(_with_balanced(4)))
    with pytest.raises(RuntimeError):
        build.check_counted_wait_kernels(
            build.resource_usage(_with_balanced(build.BALANCED_MAX_VGPR_SPILLS + 1)))
