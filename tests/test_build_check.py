"""The package build refuses kernels that need private (scratch) memory: its
parser of the compiler's per-kernel resource report (CPU only)."""
from w8a8_int8_gemm_amd import build

REPORT = """\
k.hip:10:1: remark: Function Name: _Z5good [-Rpass-analysis=kernel-resource-usage]
k.hip:10:1: remark:     VGPRs: 95 [-Rpass-analysis=kernel-resource-usage]
k.hip:10:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
k.hip:20:1: remark: Function Name: _Z3bad [-Rpass-analysis=kernel-resource-usage]
k.hip:20:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
k.hip:20:1: remark:     ScratchSize [bytes/lane]: 932 [-Rpass-analysis=kernel-resource-usage]
"""


def test_scratch_kernels_are_reported():
    assert build._scratch_kernels(REPORT) == ["_Z3bad: 932 bytes/lane"]


def test_clean_report_passes():
    assert build._scratch_kernels(REPORT.split("k.hip:20")[0]) == []


def test_report_flag_is_in_every_compile():
    assert "-Rpass-analysis=kernel-resource-usage" in build.REPORT
