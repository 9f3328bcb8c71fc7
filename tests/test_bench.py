"""Host-side checks of bench.py: the one-GPU contract and the traffic record's
source check.  No GPU is touched."""

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
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_is_reported_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    src = tmp_path / "block_gemm.hip"
    src.write_text("// kernel source\n")
    rec = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "GEMM_SOURCE", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.measured_traffic() is None                       # no record
    rec.write_text(json.dumps({"block_gemm_hip_sha256": bench.source_hash(str(src)),
                               "bytes_per_launch": 1234}))
    assert bench.measured_traffic() == 1234
    src.write_text("// kernel source, changed\n")
    assert bench.measured_traffic() is None                       # taken on another source
    rec.write_text("{not json")
    assert bench.measured_traffic() is None
