"""Host-side checks of bench.py (no GPU): the single-GPU guard and the lookup
of the committed HBM-traffic records."""
import hashlib
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
    (tmp_path / "profiles").mkdir()
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    rec = dict(kernel="k", hbm_bytes=123456.6, source="k.hip", source_sha256=sha)
    (tmp_path / "profiles" / "gemm_x_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("gemm_x") == 123457
    assert bench.measured_traffic("gemm_no_such_workload") is None
    # a record whose source has changed since the counters were taken is not used
    src.write_text("kernel v2\n")
    assert bench.measured_traffic("gemm_x") is None


def test_sample_experts():
    import numpy as np
    offs = np.concatenate([[0], np.cumsum([5, 0, 9, 2, 7, 0, 3, 4])])
    ex = bench.sample_experts(offs, 5, seed=1)
    assert len(ex) == 5 and ex == sorted(ex)
    assert {2, 3} <= set(ex)                # largest (9 rows) and smallest non-empty (2)
    assert not {1, 5} & set(ex)             # empty experts are never sampled
    assert bench.sample_experts(offs, 99, seed=1) == [0, 2, 3, 4, 6, 7]
    assert bench.sample_experts(offs, 5, seed=1) == bench.sample_experts(offs, 5, seed=1)
