"""Host-side checks of bench.py (CPU only): the one-GPU rule, the CPU
baseline's record, and that the committed GEMM byte counters belong to the
GEMM source in the tree (bench.py reports roofline.traffic only then)."""
import json
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_cpu_baseline_record_on_the_tiny_workload():
    wl = synth.WORKLOADS["tiny"]
    inp = synth.make_inputs(wl)
    r = bench.cpu_baseline(inp, wl, 0.2)
    assert r["kind"] == "oracle" and r["unit"] == "TOPS"
    assert r["value"] > 0 and r["cores"] >= 1 and r["passes"] >= 1
    assert r["seconds"] > 0 and "pass" in r["sample"]


def test_committed_gemm_counters_match_the_gemm_source():
    with open(bench.COUNTERS) as f:
        rec = json.load(f)
    assert rec["kernel_source_sha256_16"] == bench._kernel_hash(), (
        "k_gemm.hip changed since the FETCH_SIZE / WRITE_SIZE passes: retake them")
    assert rec["hbm_bytes_per_launch"] > 112 * 2**20   # at least the algorithmic bytes


def test_clock_fields_from_the_counter_record(monkeypatch):
    """The roofline's clock fields: the INT8 peak scaled to the observed shader
    clock, and the run's fraction of it; absent record -> sclk_ghz None."""
    import bench
    monkeypatch.setattr(bench, "_counters", lambda: {"sclk_ghz": 1.8, "mfma_busy": 0.67})
    f = bench._clock_fields(2250.0)
    assert abs(f["peak_at_sclk"] - 5000.0 * 1.8 / 2.4) < 1e-9
    assert abs(f["frac_at_sclk"] - 2250.0 / 3750.0) < 1e-12
    assert f["mfma_busy"] == 0.67
    monkeypatch.setattr(bench, "_counters", lambda: {})
    assert bench._clock_fields(2250.0) == {"sclk_ghz": None}


def test_committed_counter_record_has_a_plausible_clock():
    import bench
    c = bench._counters()
    assert 1.0 < c["sclk_ghz"] <= bench.PEAK_SCLK_GHZ
    assert 0.0 < c["mfma_busy"] <= 1.0


def test_rocpd_summary_trace_table(tmp_path, capsys):
    """The kernel-trace summary: calls, mean, min, max and median per kernel,
    slowest total first (a database with the kernels view rocprofv3 writes)."""
    import sqlite3
    import bench
    db = tmp_path / "t.db"
    con = sqlite3.connect(db)
    con.execute("create table k(name text, duration real)")
    con.executemany("insert into k values (?, ?)",
                    [("a", 1000.0), ("a", 3000.0), ("a", 2600.0), ("b", 500.0), ("b", 700.0)])
    con.execute("create view kernels as select * from k")
    con.commit()
    con.close()
    bench.rocpd_summary(str(db))
    lines = capsys.readouterr().out.splitlines()
    assert lines[1].split()[-1] == "median_us"
    a = lines[2].split()
    assert a[0] == "a" and a[1:] == ["3", "2.20", "1.00", "3.00", "2.60"]
    b = lines[3].split()
    assert b[0] == "b" and b[1:] == ["2", "0.60", "0.50", "0.70", "0.60"]
