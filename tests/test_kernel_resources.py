"""Per-kernel register and memory resources of the built library (CPU only:
the compiler's kernel-resource-usage report, which the build records).

Every kernel of libqmv must run without scratch memory (no register spills,
no private arrays in memory), use no accumulation registers (the matrix-core
kernels are built to keep their results in VGPRs), spill no scalar
registers, and fit at least two waves per SIMD."""
import json
import os

import pytest

from quant_mat_vec_amd import build


@pytest.fixture(scope="module")
def kernels():
    if not os.path.exists(build.RESOURCES) or not os.path.exists(build.LIB):
        build.build(verbose=False)
    with open(build.RESOURCES) as f:
        ks = json.load(f)
    assert ks, "no kernel resource report"
    return ks


def test_every_source_reports_kernels(kernels):
    srcs = {os.path.basename(s) for s in build.sources()} - {"api.hip"}     # api.hip: host code only
    assert {k["source"] for k in kernels} == srcs
    for k in kernels:
        for field in ("vgprs", "agprs", "scratch_bytes_per_lane", "occupancy_waves_per_simd", "sgpr_spill",
                      "vgpr_spill"):
            assert field in k, (k["kernel"], field)


def test_no_scratch_spills_or_accumulation_registers(kernels):
    bad = [(k["kernel"], k["scratch_bytes_per_lane"], k["vgpr_spill"], k["sgpr_spill"]) for k in kernels
           if k["scratch_bytes_per_lane"] or k["vgpr_spill"] or k["sgpr_spill"]]
    assert not bad, bad
    bad = [(k["kernel"], k["agprs"]) for k in kernels if k["agprs"]]
    assert not bad, bad


def test_at_least_two_waves_per_simd(kernels):
    bad = [(k["kernel"], k["vgprs"], k["occupancy_waves_per_simd"]) for k in kernels
           if k["occupancy_waves_per_simd"] < 2]
    assert not bad, bad
