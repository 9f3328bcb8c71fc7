"""The decode kernels' workgroup width across weight widths.

The decode kernel (M <= 32) launches one to five compute waves per workgroup,
and the wide decode kernel (32 < M <= 64) one to five weight tiles, the fewest
that keep the grid within one workgroup per CU: on a 256-CU device, one up to
N = 4096, two up to 8192, three up to 12288, four up to 16384 and five above.
Cases sit on both sides of every boundary, with one and two activation row
tiles (M <= 16, 17..32) and three and four in the wide kernel (33..48, 49..64),
K / 128 a multiple of 4 or not (scale table or per-block scales), both scale
formats and both output dtypes, and must meet the oracle's bound on every
element.  Inputs follow the GEMM recipe (normal
activations with outliers, E4M3 weight codes, log-uniform block scales).
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as fb
import oracle
from inputs import gen
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

CASES = [  # m, n, k, scale_fmt, out
    (1, 4096, 512, None, "bf16"),
    (17, 4097, 640, "ue8m0", "f32"),
    (32, 7168, 512, None, "f32"),
    (5, 8192, 640, "ue8m0", "bf16"),
    (16, 8193, 512, None, "bf16"),
    (20, 12288, 640, None, "bf16"),
    (2, 12289, 512, "ue8m0", "f32"),
    (31, 16384, 512, "ue8m0", "bf16"),
    (8, 16385, 640, None, "f32"),
    (33, 4096, 512, "ue8m0", "bf16"),
    (48, 4097, 640, None, "f32"),
    (64, 8193, 512, None, "bf16"),
    (40, 12289, 640, "ue8m0", "f32"),
    (64, 16384, 512, "ue8m0", "bf16"),
    (49, 16385, 640, None, "bf16"),
]


@pytest.mark.parametrize("m,n,k,fmt,out", CASES)
def test_decode_width(m, n, k, fmt, out):
    G.announce(f"decode width m={m} n={n} k={k} scale_fmt={fmt} out={out}")
    d = gen.custom_gemm(seed=8000 + n + 100000 * m, m=m, n=n, k=k, outliers=True)
    dev = G.device()
    y, s = fb.act_quant(d["x"].to(dev), 128, fmt)
    w = torch.from_numpy(d["w"]).to(dev)
    ws = torch.from_numpy(d["w_s"]).to(dev)
    c = fb.fp8_gemm(y, s, w, ws, torch.bfloat16 if out == "bf16" else torch.float32, fmt)
    got = c.float().cpu().numpy().astype(np.float64)
    aq, as_ = oracle.act_quant(d["x"].float().numpy(), 128, fmt)
    ref = oracle.fp8_gemm(aq, as_, d["w"], d["w_s"])
    ok = oracle.gemm_check(got, ref, oracle.gemm_tolerance(aq, as_, d["w"], d["w_s"]), out)
    assert ok.all(), f"{int((~ok).sum())} of {ok.size} outside the oracle bound"
