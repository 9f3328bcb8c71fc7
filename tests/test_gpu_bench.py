"""bench.py's JSON line, from a two-step run in this process."""

import json
import sys

import pytest

import bench
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def test_bench_line(monkeypatch, capsys):
    G.announce("bench.py --steps 2 --warmup 1 --no-cpu")
    monkeypatch.setattr(sys, "argv", ["bench.py", "--steps", "2", "--warmup", "1", "--no-cpu"])
    bench.main()
    rec = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 2 and rec["warmup"] == 1
    assert rec["higher_is_better"] is True and rec["cpu_baseline"] is None
    assert "workload" in rec["config"]
    # whole-step throughput from the step time
    assert rec["value"] == pytest.approx(bench.GEMM_FLOP / (rec["ms_per_step"] * 1e-3) / 1e12)
    roof = rec["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 5000.0
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"])
    assert 0.0 < roof["frac"] < 1.0
    # the GEMM alone is faster than the whole step
    assert roof["achieved"] > rec["value"]
    kern = rec["kernels"]
    total_us = kern["act_quant"]["us"] + kern["weight_dequant"]["us"] + kern["block_gemm"]["us"]
    assert 0.0 < total_us <= rec["ms_per_step"] * 1e3 * 1.05
