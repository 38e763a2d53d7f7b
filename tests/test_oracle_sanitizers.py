"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer and
run once through every step on ragged shapes (CPU only): any out-of-bounds
access, leak or undefined arithmetic in the oracle fails this test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_san"
    cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-ffp-contract=off", "-std=c11",
           os.path.join(ROOT, "oracle", "sq_oracle.c"),
           os.path.join(ROOT, "oracle", "sanitize_driver.c"), "-o", str(exe), "-lm", "-fopenmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "oracle sanitizer run ok" in r.stdout, r.stdout + r.stderr
