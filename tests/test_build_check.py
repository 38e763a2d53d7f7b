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


def test_inline_asm_outputs_are_early_clobber():
    """Every inline-asm statement in the kernels that issues more than one
    instruction and has VGPR outputs declares them early-clobber ("=&v").
    Without it the compiler may give an earlier load's destination the
    register a later load of the same statement still takes its address
    from, and a load that lands early redirects the later one."""
    import glob
    import os
    import re
    stmt = re.compile(r"asm\s+volatile\s*\((.*?)\)\s*;", re.S)
    bad = []
    for path in sorted(glob.glob(os.path.join(build.CSRC, "*.hip"))):
        src = open(path).read()
        for m in stmt.finditer(src):
            # the template's string literals, then ": outputs : inputs ..."
            t = re.match(r'\s*((?:"(?:[^"\\]|\\.)*"\s*)+)(.*)$', m.group(1), re.S)
            if t is None or "\\n" not in t.group(1) or not t.group(2).startswith(":"):
                continue
            outputs = t.group(2)[1:].split(":")[0]
            if re.search(r'"=v"', outputs):
                line = src.count("\n", 0, m.start()) + 1
                bad.append(f"{os.path.basename(path)}:{line}")
    assert bad == [], bad
