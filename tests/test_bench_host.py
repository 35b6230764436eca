"""Host-side checks of bench.py (no GPU): the single-GPU guard and the lookup
of the committed HBM-traffic records."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_record_lookup(tmp_path, monkeypatch):
    # the committed records describe the current GEMM source
    rec = json.load(open(os.path.join(
        ROOT, "profiles", "gemm_gate_up_moe_ffn_e128_top8_t4096_h2048_i768_traffic.json")))
    got = bench.measured_traffic("gemm_gate_up_moe_ffn_e128_top8_t4096_h2048_i768")
    assert got == int(round(rec["hbm_bytes"]))
    assert bench.measured_traffic("gemm_no_such_workload") is None
    # a record whose source has changed since the counters were taken is not used
    (tmp_path / "profiles").mkdir()
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    stale = dict(rec, source="k.hip", source_sha256="0" * 64)
    (tmp_path / "profiles" / "gemm_x_traffic.json").write_text(json.dumps(stale))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("gemm_x") is None
