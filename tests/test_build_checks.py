"""The build's guard against kernels that use scratch memory (sparse_embedding_lookup_amd/build.py):
it reads hipcc's kernel-resource-usage remarks and names every kernel whose ScratchSize is not 0."""
from sparse_embedding_lookup_amd import build

REPORT = """\
a.hip:10:1: remark: Function Name: _Z6kernelv [-Rpass-analysis=kernel-resource-usage]
a.hip:10:1: remark:     VGPRs: 125 [-Rpass-analysis=kernel-resource-usage]
a.hip:10:1: remark:     ScratchSize [bytes/lane]: 272 [-Rpass-analysis=kernel-resource-usage]
a.hip:20:1: remark: Function Name: _Z5cleanv [-Rpass-analysis=kernel-resource-usage]
a.hip:20:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_scratch_kernels_named():
    assert build._scratch_kernels(REPORT) == ["_Z6kernelv (272 bytes per lane)"]


def test_no_scratch_no_names():
    assert build._scratch_kernels(REPORT.replace("272", "0")) == []
    assert build._scratch_kernels("") == []
