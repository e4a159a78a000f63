"""The build's reading of the compiler's resource-usage remarks: the parser, the
scratch check built on it, and the table the build writes beside its objects."""

import os

import pytest

from residual_add_rmsnorm_fp32_amd import build

REMARKS = """\
x.hpp:1:1: remark: Function Name: _ZN3far14far_vec_kernelINS_4Bf16ELi2ELi5ELi2ELb0ELb1EEEvNS_10KernelArgsEii [-Rpass-analysis=kernel-resource-usage]
x.hpp:1:1: remark:     TotalSGPRs: 91 [-Rpass-analysis=kernel-resource-usage]
x.hpp:1:1: remark:     VGPRs: 126 [-Rpass-analysis=kernel-resource-usage]
x.hpp:1:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]
x.hpp:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hpp:1:1: remark:     Occupancy [waves/SIMD]: 4 [-Rpass-analysis=kernel-resource-usage]
x.hpp:1:1: remark:     LDS Size [bytes/block]: 256 [-Rpass-analysis=kernel-resource-usage]
x.hpp:1:1: remark: Function Name: spilling_kernel [-Rpass-analysis=kernel-resource-usage]
x.hpp:1:1: remark:     VGPRs: 128 [-Rpass-analysis=kernel-resource-usage]
x.hpp:1:1: remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=kernel-resource-usage]
"""


def test_remarks_parsed_per_kernel():
    rows = dict(build._resources(REMARKS))
    first = rows["_ZN3far14far_vec_kernelINS_4Bf16ELi2ELi5ELi2ELb0ELb1EEEvNS_10KernelArgsEii"]
    assert first == {"sgprs": 91, "vgprs": 126, "agprs": 0, "scratch": 0, "waves_per_simd": 4,
                     "lds_bytes": 256}
    assert rows["spilling_kernel"] == {"vgprs": 128, "scratch": 16}


def test_scratch_is_a_build_error():
    with pytest.raises(RuntimeError, match="spilling_kernel"):
        build._check_no_scratch(REMARKS, "x.o")
    build._check_no_scratch(REMARKS.split("x.hpp:1:1: remark: Function Name: spilling")[0], "x.o")


def test_resource_table_of_the_build():
    if not os.path.exists(build.RESOURCES_PATH):
        pytest.skip("no build in this tree: run __graft_entry__.build() first")
    lines = open(build.RESOURCES_PATH).read().splitlines()
    assert lines[0].split("\t") == ["kernel", "sgprs", "vgprs", "agprs", "scratch", "waves_per_simd",
                                    "lds_bytes"]
    fused = [l.split("\t") for l in lines[1:] if "far_vec_kernel" in l]
    assert len(fused) > 100
    for row in fused:
        assert row[4] == "0", row
        # every fused kernel fits the 1024-thread launch bound's register budget
        assert 0 < int(row[2]) <= 128, row
