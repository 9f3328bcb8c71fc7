"""bench.py's JSON line, from short runs in this process."""

import json
import sys

import pytest

import bench
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def test_bench_line(monkeypatch, capsys):
    G.announce("bench.py --steps 2 --warmup 1 --no-cpu --no-configs")
    bench.main(["--steps", "2", "--warmup", "1", "--no-cpu", "--no-configs"])
    rec = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 2 and rec["warmup"] == 1
    assert rec["higher_is_better"] is True and rec["cpu_baseline"] is None
    assert "workload" in rec["config"] and "configs" not in rec
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


def test_bench_configs_records():
    G.announce("bench.bench_configs, 2 launches each, no oracle")
    import torch
    args = bench.parse(["--config-reps", "2", "--no-cpu"])
    recs = bench.bench_configs(args, torch.cuda.current_stream())
    expect = {"tiny", "act_quant_none", "act_quant_ue8m0", "dequant", "dequant_ragged", "weight_quant_none",
              "weight_quant_ue8m0", "decode_m1", "decode_m8", "decode_m32", "decode_m64", "prefill_shape1",
              "prefill_shape2"}
    assert set(recs) == expect
    for key in expect - {"tiny"}:
        r = recs[key]
        assert r["us"] > 0 and "workload" in r, key
        if "frac_hbm" in r:
            assert r["GB/s"] == pytest.approx(r["bytes"] / (r["us"] * 1e-6) / 1e9)
            assert 0 < r["frac_hbm"] < 1.5, key
            if not key.startswith("decode"):
                assert r["rotation"] * r["bytes"] >= bench.ROTATE_BYTES, key
        else:
            assert 0 < r["frac_mfma"] < 1, key
    assert recs["dequant_ragged"]["bytes"] == 396566240 and recs["dequant"]["bytes"] == 396393984
    assert recs["act_quant_none"]["bytes"] == 177995776
