"""A seeded sweep of GEMM shapes across every kernel-selection boundary.

Row counts sit on both sides of each boundary of the dispatch (16/17 and
32/33 rows: decode kernel tile counts; 32/33 and 64/65: decode, wide decode and
tiled kernels; 255-257: one or two tile rows), with N and K drawn at random
(N from 1 to 1,300, K a multiple of 128 up to 3,072, so edge tiles, single K
blocks and K / 128 not a multiple of 4 all occur).  Each case goes through
fp8_gemm (split-K allowed) with act_quant's activations in both scale formats
and both output dtypes, and must meet the oracle's bound on every element.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as fb
import oracle
from inputs import gen
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

ROWS = [1, 2, 3, 15, 16, 17, 31, 32, 33, 47, 48, 63, 64, 65, 66, 127, 128, 129, 255, 256, 257, 300, 511, 640]


def _cases():
    rng = np.random.default_rng(2024)
    out = []
    for i, m in enumerate(ROWS):
        n = int(rng.integers(1, 1301))
        k = 128 * int(rng.integers(1, 25))
        fmt = (None, "ue8m0")[i % 2]
        dtype = ("bf16", "f32")[(i // 2) % 2]
        out.append((m, n, k, fmt, dtype))
    return out


@pytest.mark.parametrize("m,n,k,fmt,out", _cases())
def test_shape_sweep(m, n, k, fmt, out):
    G.announce(f"gemm sweep m={m} n={n} k={k} scale_fmt={fmt} out={out}")
    d = gen.custom_gemm(seed=7000 + m, m=m, n=n, k=k, outliers=True)
    dev = G.device()
    y, s = fb.act_quant(d["x"].to(dev), 128, fmt)
    w = torch.from_numpy(d["w"]).to(dev)
    ws = torch.from_numpy(d["w_s"]).to(dev)
    c = fb.fp8_gemm(y, s, w, ws, torch.bfloat16 if out == "bf16" else torch.float32, fmt)
    got = c.float().cpu().numpy().astype(np.float64)
    aq, as_ = oracle.act_quant(d["x"].float().numpy(), 128, fmt)
    assert np.array_equal(y.view(torch.uint8).cpu().numpy(), aq)
    ref = oracle.fp8_gemm(aq, as_, d["w"], d["w_s"])
    ok = oracle.gemm_check(got, ref, oracle.gemm_tolerance(aq, as_, d["w"], d["w_s"]), out)
    assert ok.all(), f"{int((~ok).sum())} of {ok.size} outside the oracle bound"
