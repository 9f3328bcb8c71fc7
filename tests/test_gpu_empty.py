"""Empty inputs on the GPU: calls whose outputs have no elements.

A batch with no rows (an expert that receives no tokens, an empty decode
batch) is an ordinary input.  Through the binding every entry point returns
outputs of the right shapes and dtypes, queues no kernel for them, and leaves
the stream usable: a real call right after each empty one still matches the
oracle.  act_quant_gemm with no weight rows still quantizes x, bit-identically
to act_quant.  A product with K = 0 is rejected rather than returning
uninitialized memory.  Entry points called through the C ABI with a zero size
return FP8BSQ_OK with NULL pointers.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as fb
import oracle
from fp8_block_scaled_quant_amd import _lib
from inputs import gen
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _real_act_quant_check(dev):
    """A non-empty act_quant after the empty calls, against the oracle."""
    x = gen.act_quant_workload(m=4, k=512, seed=77)["x"]
    y, s = fb.act_quant(x.to(dev))
    wq, ws = oracle.act_quant(x.float().numpy(), 128, None)
    assert np.array_equal(y.view(torch.uint8).cpu().numpy(), wq)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), ws.view(np.uint32))


@pytest.mark.parametrize("shape", [(0, 7168), (2, 0, 512), (4, 0)])
def test_act_quant_empty(shape):
    G.announce(f"empty act_quant {shape}")
    dev = G.device()
    for dt in (torch.bfloat16, torch.float32):
        x = torch.empty(shape, dtype=dt, device=dev)
        for fmt in (None, "ue8m0"):
            y, s = fb.act_quant(x, 128, fmt)
            assert y.dtype == torch.float8_e4m3fn and tuple(y.shape) == shape
            assert s.dtype == torch.float32 and tuple(s.shape) == shape[:-1] + (shape[-1] // 128,)
    torch.cuda.synchronize()
    _real_act_quant_check(dev)


@pytest.mark.parametrize("m,n", [(0, 300), (300, 0), (0, 0)])
def test_weight_dequant_and_quant_empty(m, n):
    G.announce(f"empty weight_dequant/weight_quant {m}x{n}")
    dev = G.device()
    grid = (-(-m // 128), -(-n // 128))
    codes = torch.empty((m, n), dtype=torch.uint8, device=dev)
    scales = torch.empty(grid, dtype=torch.float32, device=dev)
    for out in (torch.bfloat16, torch.float32):
        y = fb.weight_dequant(codes, scales, 128, out)
        assert y.dtype == out and tuple(y.shape) == (m, n)
    w = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    q, s = fb.weight_quant(w, 128, "ue8m0")
    assert tuple(q.shape) == (m, n) and tuple(s.shape) == grid
    torch.cuda.synchronize()
    _real_act_quant_check(dev)


@pytest.mark.parametrize("m,n", [(0, 256), (16, 0), (0, 0)])
def test_gemm_empty(m, n):
    G.announce(f"empty fp8_gemm {m}x{n}x512")
    dev = G.device()
    k = 512
    a = torch.empty((m, k), dtype=torch.uint8, device=dev)
    a_s = torch.empty((m, k // 128), dtype=torch.float32, device=dev)
    b = torch.empty((n, k), dtype=torch.uint8, device=dev)
    b_s = torch.empty((-(-n // 128), k // 128), dtype=torch.float32, device=dev)
    for fmt in (None, "ue8m0"):
        for split in (True, False):
            c = fb.fp8_gemm(a, a_s, b, b_s, torch.float32, fmt, split)
            assert c.dtype == torch.float32 and tuple(c.shape) == (m, n)
    c3 = fb.fp8_gemm(a.view(1, m, k), a_s.view(1, m, k // 128), b, b_s)
    assert tuple(c3.shape) == (1, m, n)
    torch.cuda.synchronize()
    d = gen.custom_gemm(seed=90, m=3, n=200, k=k)
    x = d["x"].to(dev)
    y, s = fb.act_quant(x)
    c = fb.fp8_gemm(y, s, torch.from_numpy(d["w"]).to(dev), torch.from_numpy(d["w_s"]).to(dev), torch.float32)
    wq, ws = oracle.act_quant(d["x"].float().numpy(), 128, None)
    ref = oracle.fp8_gemm(wq, ws, d["w"], d["w_s"])
    ok = oracle.gemm_check(c.cpu().numpy(), ref, oracle.gemm_tolerance(wq, ws, d["w"], d["w_s"]), "f32")
    assert ok.all()


def test_gemm_rejects_k_zero():
    dev = G.device()
    a = torch.empty((4, 0), dtype=torch.uint8, device=dev)
    a_s = torch.empty((4, 0), dtype=torch.float32, device=dev)
    b = torch.empty((8, 0), dtype=torch.uint8, device=dev)
    b_s = torch.empty((1, 0), dtype=torch.float32, device=dev)
    with pytest.raises(ValueError):
        fb.fp8_gemm(a, a_s, b, b_s)
    with pytest.raises(ValueError):
        fb.act_quant_gemm(torch.empty((4, 0), dtype=torch.bfloat16, device=dev), b, b_s)


@pytest.mark.parametrize("m", [1, 40])
def test_act_quant_gemm_without_weight_rows(m):
    """n = 0: c is [m, 0]; y and s are still act_quant's, bit for bit."""
    G.announce(f"act_quant_gemm m={m} n=0")
    dev = G.device()
    x_cpu = gen.act_quant_workload(m=m, k=1024, seed=80 + m)["x"]
    x = x_cpu.to(dev)
    b = torch.empty((0, 1024), dtype=torch.float8_e4m3fn, device=dev)
    b_s = torch.empty((0, 8), dtype=torch.float32, device=dev)
    bias = torch.empty((0,), dtype=torch.bfloat16, device=dev)
    for fmt in (None, "ue8m0"):
        c, y, s = fb.act_quant_gemm(x, b, b_s, fmt, torch.bfloat16, bias)
        assert tuple(c.shape) == (m, 0)
        y2, s2 = fb.act_quant(x, 128, fmt)
        assert torch.equal(y.view(torch.uint8), y2.view(torch.uint8)) and torch.equal(s, s2)
        wq, ws = oracle.act_quant(x_cpu.float().numpy(), 128, fmt)
        assert np.array_equal(y.view(torch.uint8).cpu().numpy(), wq)
        assert np.array_equal(s.cpu().numpy().view(np.uint32), ws.view(np.uint32))


def test_act_quant_gemm_and_linear_with_no_rows():
    G.announce("act_quant_gemm m=0, Linear on an empty batch")
    dev = G.device()
    d = gen.custom_gemm(seed=91, m=1, n=300, k=512)
    w = torch.from_numpy(d["w"]).to(dev)
    ws = torch.from_numpy(d["w_s"]).to(dev)
    x = torch.empty((0, 512), dtype=torch.bfloat16, device=dev)
    c, y, s = fb.act_quant_gemm(x, w, ws)
    assert tuple(c.shape) == (0, 300) and tuple(y.shape) == (0, 512) and tuple(s.shape) == (0, 4)
    lin = fb.Linear(512, 300, bias=True, device=dev)
    out = lin(torch.empty((2, 0, 512), dtype=torch.bfloat16, device=dev))
    assert tuple(out.shape) == (2, 0, 300) and out.dtype == torch.bfloat16
    torch.cuda.synchronize()
    _real_act_quant_check(dev)


def test_c_abi_zero_sizes_with_null_pointers():
    G.device()
    lib = _lib.lib()
    st = G.stream()
    N = None
    assert lib.fp8_act_quant(N, _lib.BF16, 0, 7168, 128, _lib.SCALE_NONE, N, N, st) == _lib.OK
    assert lib.fp8_weight_dequant(N, N, 0, 7168, 128, N, _lib.BF16, st) == _lib.OK
    assert lib.fp8_weight_quant(N, _lib.BF16, 18432, 0, 128, _lib.SCALE_UE8M0, N, N, st) == _lib.OK
    assert lib.fp8_block_gemm(N, N, N, N, N, _lib.BF16, 0, 18432, 7168, st) == _lib.OK
    assert lib.fp8_block_gemm_split_noalloc(N, N, N, N, N, _lib.BF16, 8192, 0, 7168, 1, st) == _lib.OK
    assert lib.fp8_act_quant_gemm(N, _lib.BF16, 0, N, N, N, N, _lib.BF16, 0, 18432, 7168, N, N, st) == _lib.OK
    assert lib.fp8_block_gemm_split_workspace(0, 18432, 7168) == 0
    torch.cuda.synchronize()
    _real_act_quant_check(G.device())
