"""GPU parity for fp8_block_gemm against the float64 oracle.

Bound (per element): |gpu - C| <= 1e-3 * sum_k |a_k b_k| for FP32 output,
plus one bf16 ulp of C for BF16 output; NaN/Inf always fail.

Cases: the tiny workload (fp32 activations [16, 512] quantized by the GPU
act_quant, weights [256, 512], fp32 out); the decode workloads (M = 1, 8, 32
through the decode kernel, and 33, 48 and 64 through the wide kernel, whose
waves each run one activation tile against five weight tiles; N = 18432,
K = 7168, bf16 out), checked on every element; both prefill
shapes at full size (M = 8192) checked on sampled rows (first, last and 512
random rows, every column); ragged shapes with partial tiles in M and N.
"""

import numpy as np
import pytest
import torch

import oracle
from inputs import gen
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _assert_close(got, a, a_s, b, b_s, out, rows=None, label=""):
    c = oracle.fp8_gemm(a, a_s, b, b_s, rows=rows)
    tol = oracle.gemm_tolerance(a, a_s, b, b_s, rows=rows)
    ok = oracle.gemm_check(got, c, tol, out)
    if not ok.all():
        bad = np.argwhere(~ok)
        i, j = bad[0]
        raise AssertionError(f"{label}: {len(bad)} elements out of bound; first ({i},{j}) "
                             f"gpu={got[i, j]!r} oracle={c[i, j]!r} tol={tol[i, j]!r}")
    return c


def _quantized_activations(x_cpu, scale_fmt):
    """GPU act_quant of x, checked bit-exact against the oracle's codes."""
    codes, scales = G.act_quant(x_cpu.to(G.device()), scale_fmt)
    wq, ws = oracle.act_quant(x_cpu.float().numpy(), 128, scale_fmt)
    assert np.array_equal(codes, wq) and np.array_equal(scales.view(np.uint32), ws.view(np.uint32))
    return codes, scales


def test_tiny_workload_fp32_out():
    d = gen.tiny_gemm()
    G.announce("gemm tiny 16x256x512 f32")
    a, a_s = _quantized_activations(d["x"], None)
    got = G.block_gemm(a, a_s, d["w"], d["w_s"], "f32")
    _assert_close(got, a, a_s, d["w"], d["w_s"], "f32", label="tiny")


@pytest.mark.parametrize("m", [1, 8, 32, 33, 48, 64])
def test_decode_workloads(m):
    d = gen.decode_gemm(m)
    G.announce(f"gemm decode M={m} N=18432 K=7168 bf16")
    a, a_s = _quantized_activations(d["x"], None)
    got = G.block_gemm(a, a_s, d["w"], d["w_s"], "bf16")
    _assert_close(got, a, a_s, d["w"], d["w_s"], "bf16", label=f"decode M={m}")


@pytest.mark.parametrize("shape", [1, 2])
def test_prefill_workloads_sampled_rows(shape):
    d = gen.prefill_gemm(shape)
    m = d["x"].shape[0]
    G.announce(f"gemm prefill shape {shape} M={m} N={d['w'].shape[0]} K={d['w'].shape[1]} bf16")
    a, a_s = _quantized_activations(d["x"], "ue8m0")
    got = G.block_gemm(a, a_s, d["w"], d["w_s"], "bf16")
    rng = np.random.default_rng(100 + shape)
    rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, 512, replace=False)]))
    _assert_close(got[rows], a, a_s, d["w"], d["w_s"], "bf16", rows=rows, label=f"prefill {shape}")


@pytest.mark.parametrize("m,n,k", [(1, 1, 128), (17, 200, 256), (33, 130, 384), (64, 129, 128),
                                   (100, 300, 1024), (130, 64, 640), (257, 385, 512),
                                   (40, 100, 21504), (5, 70, 20608), (20, 300, 1536), (49, 81, 2048),
                                   (56, 18440, 512)])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_ragged_shapes(m, n, k, out):
    d = gen.custom_gemm(seed=m * 1000 + n + k, m=m, n=n, k=k, outliers=True)
    G.announce(f"gemm ragged m={m} n={n} k={k} {out}")
    a, a_s = _quantized_activations(d["x"], None)
    got = G.block_gemm(a, a_s, d["w"], d["w_s"], out)
    _assert_close(got, a, a_s, d["w"], d["w_s"], out, label=f"ragged {m}x{n}x{k}")


def test_scale_indexing_probe():
    """Distinct power-of-two scales per (row, K block) and per weight tile: any
    mix-up of a_s / b_s indices breaks the bound."""
    m, n, k = 48, 384, 512
    rng = np.random.default_rng(42)
    a = gen.weight_codes(rng, m, k)
    b = gen.weight_codes(rng, n, k)
    a_s = (2.0 ** rng.integers(-20, 0, (m, k // 128))).astype(np.float32)
    b_s = (2.0 ** rng.integers(-20, 0, (n // 128, k // 128))).astype(np.float32)
    G.announce("gemm scale-indexing probe")
    for out in ("f32", "bf16"):
        got = G.block_gemm(a, a_s, b, b_s, out)
        _assert_close(got, a, a_s, b, b_s, out, label="scale probe")


@pytest.mark.parametrize("m", [300, 40])
@pytest.mark.parametrize("aligned", [True, False])
def test_scale_indexing_probe_tiled(m, aligned):
    """The tiled (M = 300) and staged-activation decode (M = 40) kernels with
    distinct non-power-of-two activation scales per (row, K block): K = 2560
    gives two full 8-K-block chunks of the scale table and a half-filled
    third; a_s offset by one float (not 16-byte aligned) takes the per-K-block
    scale transfers instead.  Both must meet the bound."""
    n, k = 384, 2560
    rng = np.random.default_rng(43)
    a = gen.weight_codes(rng, m, k)
    b = gen.weight_codes(rng, n, k)
    a_s = (2.0 ** rng.uniform(-20, 0, (m, k // 128))).astype(np.float32)
    b_s = (2.0 ** rng.uniform(-20, 0, (n // 128, k // 128))).astype(np.float32)
    dev = G.device()
    store = torch.zeros(m * (k // 128) + 1, dtype=torch.float32, device=dev)
    a_s_dev = (store[:-1] if aligned else store[1:]).view(m, k // 128)
    a_s_dev.copy_(torch.from_numpy(a_s))
    G.announce(f"gemm scale-indexing probe m={m}, a_s {'aligned' if aligned else 'offset by 4 bytes'}")
    got = G.block_gemm(None, None, b, b_s, "f32", a_dev=torch.from_numpy(a).to(dev), a_s_dev=a_s_dev)
    _assert_close(got, a, a_s, b, b_s, "f32", label="tiled scale probe")


@pytest.mark.parametrize("m,n,k", [(3, 200, 384), (100, 300, 1024), (257, 130, 640)])
def test_reference_kernel(m, n, k):
    """The reference-structure kernel (what shapes beyond the tiled and decode
    kernels' 32-bit offsets take), through fp8_block_gemm_reference."""
    d = gen.custom_gemm(seed=5 * m + n, m=m, n=n, k=k, outliers=True)
    G.announce(f"gemm reference kernel m={m} n={n} k={k}")
    a, a_s = _quantized_activations(d["x"], None)
    for out in ("bf16", "f32"):
        got = G.block_gemm(a, a_s, d["w"], d["w_s"], out, entry="fp8_block_gemm_reference")
        _assert_close(got, a, a_s, d["w"], d["w_s"], out, label=f"reference {m}x{n}x{k}")


def test_python_binding_end_to_end():
    from fp8_block_scaled_quant_amd import act_quant, fp8_gemm
    d = gen.custom_gemm(seed=5, m=40, n=256, k=512)
    dev = G.device()
    y, s = act_quant(d["x"].to(dev))
    w = torch.from_numpy(d["w"]).to(dev).view(torch.float8_e4m3fn)
    ws = torch.from_numpy(d["w_s"]).to(dev)
    c = fp8_gemm(y, s, w, ws, out_dtype=torch.float32).cpu().numpy().astype(np.float64)
    a, a_s = oracle.act_quant(d["x"].float().numpy())
    _assert_close(c, a, a_s, d["w"], d["w_s"], "f32", label="binding")
