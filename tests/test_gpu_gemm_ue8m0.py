"""GPU parity for fp8_block_gemm_ue8m0 (power-of-two activation scales applied
inside the MX-scaled MFMA).

Scaling by a power of two is exact, so on activations quantized with ue8m0
scales the result must be bit-identical to fp8_block_gemm's (which is held to
the oracle bound by test_gpu_gemm.py); the oracle bound is checked here too on
sampled rows.  Cases: both prefill shapes at full size, ragged tiled shapes,
activations with all-zero blocks (scale 2^-22), decode shapes (which share the
generic kernels), fp32 output, act_quant_gemm with ue8m0, and the binding.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as fb
import oracle
from inputs import gen
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _both(a, a_s, w, ws, out):
    generic = G.block_gemm(None, None, w, ws, out, a_dev=a, a_s_dev=a_s)
    mx = G.block_gemm(None, None, w, ws, out, a_dev=a, a_s_dev=a_s, ue8m0=True)
    assert np.array_equal(generic.view(np.uint64), mx.view(np.uint64)), \
        f"{int((generic != mx).sum())} outputs differ from fp8_block_gemm"
    return mx


@pytest.mark.parametrize("shape", [1, 2])
def test_prefill_workloads(shape):
    d = gen.prefill_gemm(shape)
    G.announce(f"gemm_ue8m0 prefill shape {shape}")
    dev = G.device()
    a, a_s = fb.act_quant(d["x"].to(dev), 128, "ue8m0")
    got = _both(a.view(torch.uint8), a_s, d["w"], d["w_s"], "bf16")
    rows = np.unique(np.concatenate([[0, a.shape[0] - 1],
                                     np.random.default_rng(shape).choice(a.shape[0], 512, replace=False)]))
    an, asn = a.view(torch.uint8).cpu().numpy(), a_s.cpu().numpy()
    c = oracle.fp8_gemm(an, asn, d["w"], d["w_s"], rows=rows)
    tol = oracle.gemm_tolerance(an, asn, d["w"], d["w_s"], rows=rows)
    assert oracle.gemm_check(got[rows], c, tol, "bf16").all()


# K = 2560 and 1536: several 8-K-block scale-table chunks, the last one half
# filled; K = 512: a single half-filled chunk; K = 768 and 128: K/128 not a
# multiple of 4, which takes the generic kernel.  1100 x 7168: 140 tiles,
# ragged in M, with several per XCD.
@pytest.mark.parametrize("m,n,k,out", [(100, 300, 1024, "bf16"), (257, 385, 512, "f32"),
                                       (300, 260, 2560, "bf16"), (513, 256, 1536, "f32"),
                                       (1100, 7168, 1024, "bf16"),
                                       (260, 300, 768, "bf16"),
                                       (65, 129, 128, "bf16"), (8, 500, 640, "f32")])
def test_shapes(m, n, k, out):
    d = gen.custom_gemm(seed=11 * m + n, m=m, n=n, k=k, outliers=True)
    G.announce(f"gemm_ue8m0 m={m} n={n} k={k} out={out}")
    a, a_s = fb.act_quant(d["x"].to(G.device()), 128, "ue8m0")
    got = _both(a.view(torch.uint8), a_s, d["w"], d["w_s"], out)
    an, asn = a.view(torch.uint8).cpu().numpy(), a_s.cpu().numpy()
    assert oracle.gemm_check(got, oracle.fp8_gemm(an, asn, d["w"], d["w_s"]),
                             oracle.gemm_tolerance(an, asn, d["w"], d["w_s"]), out).all()


def test_zero_blocks():
    x = gen.act_quant_workload(m=512, k=1024, seed=8)["x"]
    d = gen.custom_gemm(seed=9, m=1, n=256, k=1024)
    G.announce("gemm_ue8m0 activations with zero blocks")
    a, a_s = fb.act_quant(x.to(G.device()), 128, "ue8m0")
    assert bool((a_s == 2.0**-22).any())
    _both(a.view(torch.uint8), a_s, d["w"], d["w_s"], "bf16")


def test_act_quant_gemm_ue8m0_two_kernel_path():
    d = gen.custom_gemm(seed=21, m=200, n=640, k=2048, outliers=True)
    G.announce("act_quant_gemm ue8m0 m=200")
    dev = G.device()
    got, codes, scales = G.act_quant_gemm(d["x"].to(dev), d["w"], d["w_s"], "ue8m0", "bf16")
    ref = G.block_gemm(codes, scales, d["w"], d["w_s"], "bf16")
    assert np.array_equal(got.view(np.uint64), ref.view(np.uint64))


def test_binding():
    d = gen.custom_gemm(seed=31, m=300, n=512, k=1024)
    G.announce("fp8_gemm binding scale_fmt=ue8m0")
    dev = G.device()
    a, a_s = fb.act_quant(d["x"].to(dev), 128, "ue8m0")
    w, ws = torch.from_numpy(d["w"]).to(dev), torch.from_numpy(d["w_s"]).to(dev)
    assert torch.equal(fb.fp8_gemm(a, a_s, w, ws, scale_fmt="ue8m0"), fb.fp8_gemm(a, a_s, w, ws))


def _scales_with_strays(m, nkb, seed, stray_rows):
    """Power-of-two scales, except one entry in each of `stray_rows`: a value
    with mantissa bits, zero, a negative power of two, a subnormal."""
    rng = np.random.default_rng(seed)
    a_s = (2.0 ** rng.integers(-20, 0, (m, nkb))).astype(np.float32)
    strays = [np.float32(0.3), np.float32(0.0), np.float32(-0.125), np.float32(2.0**-130)]
    for i, r in enumerate(stray_rows):
        a_s[r, rng.integers(nkb)] = strays[i % len(strays)]
    return a_s


def _check_guarded(got, want, stray_rows):
    stray = np.zeros(got.shape[0], bool)
    stray[list(stray_rows)] = True
    assert np.isnan(got[stray]).all(), "rows with stray scales must be NaN"
    assert np.array_equal(got[~stray].view(np.uint64), want[~stray].view(np.uint64))


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_guard_marks_rows_with_stray_scales(out):
    """fp8_block_gemm_ue8m0 on the MX-scaled kernel checks its precondition:
    rows whose scales are not all positive normal powers of two come back NaN,
    the other rows bit-identical to fp8_block_gemm."""
    m, n, k = 300, 256, 1024
    rng = np.random.default_rng(61)
    a = gen.weight_codes(rng, m, k)
    b = gen.weight_codes(rng, n, k)
    b_s = gen.log_uniform_scales(rng, gen.scale_grid(n, k), -14, -2)
    stray_rows = [0, 5, 130, 255, 256, 299]
    a_s = _scales_with_strays(m, k // 128, 62, stray_rows)
    G.announce(f"gemm_ue8m0 guard m={m} n={n} k={k} {out}")
    got = G.block_gemm(a, a_s, b, b_s, out, ue8m0=True)
    want = G.block_gemm(a, a_s, b, b_s, out)
    _check_guarded(got, want, stray_rows)


def test_guard_on_split_path():
    m, n, k = 512, 1024, 8192
    rng = np.random.default_rng(63)
    a = gen.weight_codes(rng, m, k)
    b = gen.weight_codes(rng, n, k)
    b_s = gen.log_uniform_scales(rng, gen.scale_grid(n, k), -14, -2)
    stray_rows = [3, 511]
    a_s = _scales_with_strays(m, k // 128, 64, stray_rows)
    dev = G.device()
    ad, asd = torch.from_numpy(a).to(dev), torch.from_numpy(a_s).to(dev)
    G.announce(f"gemm_split ue8m0 guard m={m} n={n} k={k}")
    got, _ = G.block_gemm_split(ad, asd, b, b_s, "bf16", ue8m0=True)
    want, _ = G.block_gemm_split(ad, asd, b, b_s, "bf16", ue8m0=False)
    _check_guarded(got, want, stray_rows)
