"""The FP8 Linear module: structure on the CPU, numerics on the GPU.

GPU cases check the forward pass against the oracle composition
(weight_quant -> act_quant -> fp8_gemm in float64, plus the bias) within the
GEMM bound, and bit-identity with the underlying act_quant_gemm call; 3-D
inputs, decode (m = 1, fused path) and prefill-shaped batches, both scale
formats, fp32 output, and the dequantize-then-linear alternative.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as fb
import oracle
from inputs import gen


def test_parameters_and_shapes_cpu():
    lin = fb.Linear(1024, 4096, bias=True)
    assert lin.weight.dtype == torch.float8_e4m3fn and tuple(lin.weight.shape) == (4096, 1024)
    assert tuple(lin.weight_scale.shape) == (32, 8) and lin.weight_scale.dtype == torch.float32
    assert lin.bias.dtype == torch.bfloat16 and tuple(lin.bias.shape) == (4096,)
    assert set(lin.state_dict()) == {"weight", "weight_scale", "bias"}
    assert not any(p.requires_grad for p in lin.parameters())
    ragged = fb.Linear(256, 300)
    assert tuple(ragged.weight_scale.shape) == (3, 2) and ragged.bias is None
    with pytest.raises(ValueError):
        fb.Linear(100, 64)                      # activations need whole 1 x 128 blocks
    with pytest.raises(ValueError):
        fb.Linear(128, 64, gemm_impl="cuda")


def test_cpu_forward_raises_instead_of_falling_back():
    lin = fb.Linear(256, 128)
    with pytest.raises(ValueError):
        lin(torch.randn(2, 256, dtype=torch.bfloat16))


def _oracle_forward(x_cpu, w_cpu, bias_cpu, scale_fmt, weight_scale_fmt):
    wq, ws = oracle.weight_quant(w_cpu.float().numpy(), 128, weight_scale_fmt)
    x2 = x_cpu.float().numpy().reshape(-1, x_cpu.shape[-1])
    aq, as_ = oracle.act_quant(x2, 128, scale_fmt)
    c = oracle.fp8_gemm(aq, as_, wq, ws)
    tol = oracle.gemm_tolerance(aq, as_, wq, ws)
    if bias_cpu is not None:
        c = c + bias_cpu.float().double().numpy()[None, :]
    return c, tol, (wq, ws)


@pytest.mark.gpu
@pytest.mark.parametrize("shape,out_f,fmt,dtype,bias", [
    ((1, 7168), 18432, None, torch.bfloat16, False),        # decode, one kernel
    ((2, 3, 1024), 4096, None, torch.bfloat16, True),       # 3-D input, bias
    ((300, 1536), 2304, "ue8m0", torch.float32, True),      # ragged rows, fp32 out
    ((512, 7168), 1000, "ue8m0", torch.bfloat16, True),     # ragged N, tiled GEMM
])
def test_forward_matches_oracle(shape, out_f, fmt, dtype, bias):
    from tests import gpu_util as G
    G.announce(f"Linear x={shape} out={out_f} fmt={fmt} dtype={dtype} bias={bias}")
    dev = G.device()
    in_f = shape[-1]
    x = gen.to_bf16(np.random.default_rng(1).standard_normal(shape, dtype=np.float32))
    w = gen.weight_quant_workload(out_f, in_f, seed=out_f + in_f)["w"]
    b = gen.to_bf16(np.random.default_rng(2).standard_normal(out_f, dtype=np.float32)).to(dtype) if bias else None
    lin = fb.Linear.from_weight(w.to(dev), None if b is None else b.to(dev), scale_fmt=fmt, dtype=dtype)
    y = lin(x.to(dev))
    assert y.dtype == dtype and tuple(y.shape) == shape[:-1] + (out_f,)
    c, tol, (wq, ws) = _oracle_forward(x, w, b, fmt, None)
    assert np.array_equal(lin.weight.view(torch.uint8).cpu().numpy(), wq)
    assert np.array_equal(lin.weight_scale.cpu().numpy().view(np.uint32), ws.view(np.uint32))
    got = y.float().double().cpu().numpy().reshape(c.shape)
    ok = oracle.gemm_check(got, c, tol, "bf16" if dtype == torch.bfloat16 else "f32")
    assert ok.all(), f"{int((~ok).sum())} outputs out of the bound"
    c2, _, _ = fb.act_quant_gemm(x.to(dev), lin.weight, lin.weight_scale, fmt, dtype, lin.bias)
    assert torch.equal(y, c2)


@pytest.mark.gpu
def test_dequant_alternative():
    from tests import gpu_util as G
    G.announce("Linear gemm_impl=dequant 64x1024 -> 512")
    dev = G.device()
    x = gen.to_bf16(np.random.default_rng(3).standard_normal((64, 1024), dtype=np.float32))
    w = gen.weight_quant_workload(512, 1024, seed=4)["w"]
    lin = fb.Linear.from_weight(w.to(dev), gemm_impl="dequant", dtype=torch.float32)
    y = lin(x.to(dev)).double().cpu().numpy()
    wq, ws = oracle.weight_quant(w.float().numpy(), 128, None)
    wd = oracle.weight_dequant(wq, ws, 128, out="f32").astype(np.float64)
    ref = x.float().double().numpy() @ wd.T
    # fp32 GEMM of exact bf16 x and fp32 weights: a few fp32 roundings per output
    scale = np.abs(x.float().double().numpy()) @ np.abs(wd).T
    assert np.all(np.abs(y - ref) <= 1e-5 * scale + 1e-30)
