"""Host-side checks of the build script: the scratch-memory guard reads
hipcc's resource-usage remarks correctly."""
from ternary_weight_w1_amd import build

REMARKS = """\
a.hip:10:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]
a.hip:10:1: remark:     VGPRs: 126 [-Rpass-analysis=kernel-resource-usage]
a.hip:10:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
a.hip:20:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]
a.hip:20:1: remark:     VGPRs: 197 [-Rpass-analysis=kernel-resource-usage]
a.hip:20:1: remark:     ScratchSize [bytes/lane]: 100 [-Rpass-analysis=kernel-resource-usage]
a.hip:30:1: remark: Function Name: kern_c [-Rpass-analysis=kernel-resource-usage]
a.hip:30:1: remark:     ScratchSize [bytes/lane]: 4 [-Rpass-analysis=kernel-resource-usage]
"""


def test_spilling_kernels_names_each_kernel_with_scratch():
    assert build.spilling_kernels(REMARKS) == [("kern_b", 100), ("kern_c", 4)]


def test_spilling_kernels_empty_without_remarks():
    assert build.spilling_kernels("") == []
    assert build.spilling_kernels(REMARKS.replace(": 100 ", ": 0 ").replace(": 4 ", ": 0 ")) == []


def test_compile_asks_for_the_remarks():
    assert build.RESOURCE_REMARKS == "-Rpass-analysis=kernel-resource-usage"
