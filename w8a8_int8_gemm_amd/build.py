"""Build libsqw8a8.so (the gfx950 kernels + the C ABI) in-tree with hipcc.

    python -m w8a8_int8_gemm_amd.build            # compile every source
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsqw8a8.so")
OBJ_DIR = os.path.join(PKG, "_build")

SOURCES = ["sq_w8a8.hip", "k_calib.hip", "k_weight.hip", "k_actquant.hip", "k_gemm.hip",
           "k_gemm_decode.hip", "k_gptq.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -ffp-contract=off: no fused multiply-add anywhere (the epilogue and the
#   quantizer must round every product and sum on its own).
# -packed-fp32-ops off: no v_pk_{add,mul,fma}_f32.
CFLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


# per-source additions: the GPTQ row and column steps unroll 64 x 64 updates
# fully (their values live in registers, indexed by the loop counters), past
# clang's default cost limit for an unroll pragma
EXTRA = {"k_gptq.hip": ["-mllvm", "-pragma-unroll-threshold=200000"]}


# The compiler's per-kernel resource report; a kernel that needs private
# (scratch) memory fails the build.  Such a kernel pays for its scratch setup
# at every dispatch (a GPTQ Cholesky panel that kept its 64 row values in
# scratch took 0.85 ms instead of 25 us, the FP8 GEMM with 64-byte stages 3.7 ms
# instead of 0.12 ms), so every kernel here keeps its arrays in registers.
REPORT = ["-Rpass-analysis=kernel-resource-usage"]
_NAME = re.compile(r"remark: Function Name: (\S+)")
_SCRATCH = re.compile(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)")


def _scratch_kernels(report: str) -> list[str]:
    bad, name = [], None
    for line in report.splitlines():
        m = _NAME.search(line)
        if m:
            name = m.group(1)
            continue
        m = _SCRATCH.search(line)
        if m and int(m.group(1)) > 0:
            bad.append(f"{name}: {m.group(1)} bytes/lane")
    return bad


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, src.replace(".hip", ".o"))
    cmd = [HIPCC, *CFLAGS, *EXTRA.get(src, []), *REPORT, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    bad = _scratch_kernels(r.stderr)
    if bad:
        os.remove(obj)
        raise RuntimeError(f"{src}: kernels using private (scratch) memory:\n  " + "\n  ".join(bad))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libsqw8a8.so; returns its path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
