"""GPU parity for fp8_act_quant_gemm (act_quant then the block GEMM, one call).

For bf16 activations with m <= 16 (and m * k <= 96 K codes) the whole computation runs in
one kernel (helper waves quantize x while the GEMM's waves stream the weight; past 80 K codes
through an LDS ring of K blocks); larger m and fp32 activations queue the two kernels.
Every case checks:

* the returned codes and scales are bit-identical to the oracle's act_quant;
* C is bit-identical to the two-call path (fp8_act_quant, then
  fp8_block_gemm on its outputs) -- same codes, same scales, same kernel
  arithmetic;
* C is within the oracle GEMM's bound (1e-3 * sum |a b|, + 1 bf16 ulp).

Cases: the decode workloads M = 1-4, 8, 11 (fused), 12 (fused through the ring)
and 16, 64 (two kernels), both scale formats, fp32 output, ragged N, a single
K block, the long-K decode shape (K = 18432), the longest K the fused path takes
(K / 128 = 160), the most rows it takes (16), the limits of the LDS-resident and
the ring forms, fp32 activations, and the Python binding.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as fb
import oracle
from inputs import gen
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _run(x_cpu, w, w_s, scale_fmt, out, label):
    G.announce(f"act_quant_gemm {label} x={tuple(x_cpu.shape)} {x_cpu.dtype} N={w.shape[0]} fmt={scale_fmt} out={out}")
    dev = G.device()
    x = x_cpu.to(dev)
    got, codes, scales = G.act_quant_gemm(x, w, w_s, scale_fmt, out)
    wq, ws = oracle.act_quant(x_cpu.float().numpy(), 128, scale_fmt)
    assert np.array_equal(codes, wq), "codes differ from act_quant"
    assert np.array_equal(scales.view(np.uint32), ws.view(np.uint32)), "scales differ from act_quant"
    a2, s2 = G.act_quant(x, scale_fmt)
    two_call = G.block_gemm(a2, s2, w, w_s, out)
    assert np.array_equal(got.view(np.uint64), two_call.view(np.uint64)), \
        f"{int((got != two_call).sum())} outputs differ from the two-call path"
    c = oracle.fp8_gemm(wq, ws, w, w_s)
    tol = oracle.gemm_tolerance(wq, ws, w, w_s)
    ok = oracle.gemm_check(got, c, tol, out)
    assert ok.all(), f"{int((~ok).sum())} elements out of the oracle bound"


@pytest.mark.parametrize("m", [1, 2, 3, 4, 8, 11, 12, 16, 64])
def test_decode_workloads(m):
    d = gen.decode_gemm(m)
    _run(d["x"], d["w"], d["w_s"], None, "bf16", "decode")


@pytest.mark.parametrize("m", [1, 4, 10])
def test_ue8m0_and_fp32_out(m):
    d = gen.custom_gemm(seed=50 + m, m=m, n=2304, k=7168)
    _run(d["x"], d["w"], d["w_s"], "ue8m0", "f32", "ue8m0/f32")


# fused with all of x in LDS (bf16, m <= 16, m * k <= 80 K): one K block
# (k = 128) and three; a last batch of four loads per lane that is only partly
# used (k = 18432, m = 2: 288 blocks for 44 sixteen-lane helper groups x 4);
# the longest K, at m = 4; 80 K codes at m = 5 and m = 16; every row count in
# between at a few K.  Through the ring (80 K < m * k <= 96 K): one K block
# past 80 K at m = 5 and 16, m = 12 and 13 at K = 7168, m = 5 at K = 19200,
# and 96 K codes at m = 16.  Two kernels past the limits: m = 16 with one more
# K block, m = 16 at K = 7168, m = 6 and 7 at K = 18432, m = 5 at the longest
# K, m = 17, and K / 128 = 161.  The weight widths take one to five compute waves per workgroup
# (N = 4096 and below, 7168, 10000, 13000 and 18432 on a 256-CU device).
@pytest.mark.parametrize("m,n,k", [(1, 300, 1024), (3, 129, 128), (4, 17, 256), (2, 7168, 18432), (7, 500, 640),
                                   (1, 129, 128), (2, 96, 384), (4, 300, 20480), (5, 200, 1024),
                                   (5, 200, 16384), (5, 200, 16512), (6, 130, 1024), (8, 700, 2048),
                                   (9, 257, 4096), (10, 96, 384), (11, 300, 7168), (12, 300, 7168),
                                   (13, 7168, 6144), (14, 129, 128), (15, 640, 2560), (16, 520, 5120),
                                   (16, 130, 5248), (16, 96, 128), (17, 200, 1024), (12, 700, 7168),
                                   (16, 700, 7168), (6, 300, 18432), (5, 640, 20480), (16, 130, 6144),
                                   (16, 130, 6272), (7, 96, 18432), (2, 96, 20608), (4, 10000, 1024),
                                   (9, 13000, 2048), (13, 12289, 7168), (5, 640, 19200)])
def test_shapes(m, n, k):
    d = gen.custom_gemm(seed=m * 1000 + n + k, m=m, n=n, k=k, outliers=True)
    _run(d["x"], d["w"], d["w_s"], None, "bf16", "shape")


@pytest.mark.parametrize("m", [1, 16])
def test_fp32_activations(m):
    d = gen.custom_gemm(seed=70 + m, m=m, n=512, k=1024, dtype="f32")
    _run(d["x"], d["w"], d["w_s"], None, "f32", "fp32 x")


def test_python_binding():
    d = gen.decode_gemm(2)
    G.announce("act_quant_gemm binding M=2")
    dev = G.device()
    x = d["x"].to(dev)
    w = torch.from_numpy(d["w"]).to(dev)
    ws = torch.from_numpy(d["w_s"]).to(dev)
    c, y, s = fb.act_quant_gemm(x, w, ws)
    y2, s2 = fb.act_quant(x)
    c2 = fb.fp8_gemm(y2, s2, w, ws)
    assert c.dtype == torch.bfloat16 and tuple(c.shape) == (2, 18432)
    assert torch.equal(y.view(torch.uint8), y2.view(torch.uint8)) and torch.equal(s, s2)
    assert torch.equal(c, c2)
    with pytest.raises(ValueError):
        fb.act_quant_gemm(d["x"], w, ws)      # CPU activations: no fallback


@pytest.mark.parametrize("m,n,k,out", [
    (1, 2304, 7168, "bf16"),     # one kernel
    (2, 300, 1024, "f32"),       # one kernel, ragged N
    (9, 500, 640, "bf16"),       # decode GEMM after act_quant
    (100, 384, 512, "f32"),      # tiled GEMM
    (40, 700, 1024, "bf16"),     # wide decode kernel (M > 32)
    (3, 256, 20608, "bf16"),     # long K with K/128 = 161: no scale table
])
def test_bias_in_epilogue(m, n, k, out):
    _bias_case(m, n, k, out, None)


# ue8m0 scales through the tiled GEMM: the MX-scaled kernel's epilogue, with
# ragged N and M
@pytest.mark.parametrize("m,n,k,out", [(300, 700, 1024, "bf16"), (257, 450, 512, "f32")])
def test_bias_in_epilogue_ue8m0_tiled(m, n, k, out):
    _bias_case(m, n, k, out, "ue8m0")


def _bias_case(m, n, k, out, scale_fmt):
    d = gen.custom_gemm(seed=m + n + k, m=m, n=n, k=k)
    G.announce(f"act_quant_gemm bias m={m} n={n} k={k} out={out} scale_fmt={scale_fmt}")
    dtype = torch.bfloat16 if out == "bf16" else torch.float32
    bias = torch.from_numpy(np.random.default_rng(m).standard_normal(n).astype(np.float32) * 4).to(dtype)
    got, codes, scales = G.act_quant_gemm(d["x"].to(G.device()), d["w"], d["w_s"], scale_fmt, out,
                                          bias=bias.to(G.device()))
    wq, ws = oracle.act_quant(d["x"].float().numpy(), 128, scale_fmt)
    assert np.array_equal(codes, wq) and np.array_equal(scales.view(np.uint32), ws.view(np.uint32))
    c = oracle.fp8_gemm(wq, ws, d["w"], d["w_s"]) + bias.float().double().numpy()[None, :]
    tol = oracle.gemm_tolerance(wq, ws, d["w"], d["w_s"])
    ok = oracle.gemm_check(got, c, tol, out)
    assert ok.all(), f"{int((~ok).sum())} elements out of the bound"
