"""GPU parity for fp8_act_quant: codes and scales bit-identical to the oracle.

Cases: the full bandwidth workload (bf16 [8192, 7168], 0.1% outliers x100,
one zero block per 128-row group) with both scale formats; ragged block counts
that leave partial waves and workgroups; fp32 inputs; every finite bf16 value
inside blocks with many different maxima; an encoder sweep through blocks whose
scale is exactly 1 (every fp32 value within 64 ulps of each E4M3 rounding
midpoint, fp32 subnormals, signed zeros); block maxima whose fp32 quotient
lands one ulp above 448; zero and sub-clamp blocks.
"""

import numpy as np
import pytest
import torch

import oracle
from inputs import gen
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _check(x_cpu: torch.Tensor, scale_fmt, label: str):
    G.announce(f"act_quant {label} shape={tuple(x_cpu.shape)} dtype={x_cpu.dtype} scale_fmt={scale_fmt}")
    codes, scales = G.act_quant(x_cpu.to(G.device()), scale_fmt)
    want_q, want_s = oracle.act_quant(x_cpu.float().numpy(), 128, scale_fmt)
    assert np.array_equal(scales.view(np.uint32), want_s.view(np.uint32)), \
        f"scales differ at {np.argwhere(scales.view(np.uint32) != want_s.view(np.uint32))[:5]}"
    bad = np.argwhere(codes != want_q)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:5].tolist()}"


@pytest.mark.parametrize("scale_fmt", [None, "ue8m0"])
def test_bandwidth_workload(scale_fmt):
    x = gen.act_quant_workload()["x"]
    _check(x, scale_fmt, "workload 8192x7168")


@pytest.mark.parametrize("rows,k", [(1, 128), (3, 384), (5, 7168), (17, 256), (1, 1024), (65, 128 * 7)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_block_counts(rows, k, dtype):
    x = gen.activations(gen.rng_for(1000 + rows * 7 + k), rows, k, dtype=dtype, outliers=True)
    _check(x, None, "ragged")
    _check(x, "ue8m0", "ragged")


def test_tiny_fp32_workload():
    x = gen.tiny_gemm()["x"]
    _check(x, None, "tiny fp32")
    _check(x, "ue8m0", "tiny fp32")


def _blocks_all_bf16(amaxes):
    bits = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    bits = bits[np.isfinite(bits)]
    rows = []
    for amax in amaxes:
        vals = bits[np.abs(bits) <= amax]
        nblk = -(-vals.size // 127)
        pad = np.zeros(nblk * 127, np.float32)
        pad[:vals.size] = vals
        rows.append(np.concatenate([np.full((nblk, 1), amax, np.float32), pad.reshape(nblk, 127)], 1))
    blocks = np.concatenate(rows, 0)
    nb = blocks.shape[0] - blocks.shape[0] % 8
    return blocks[:nb].reshape(-1, 1024)


@pytest.mark.parametrize("scale_fmt", [None, "ue8m0"])
def test_every_bf16_value(scale_fmt):
    rng = np.random.default_rng(77)
    amaxes = [np.float32(v) for v in (448.0, 1.0, 3.0, 0.5, 2.0**-20, 7e-5, 1e4, 3.3e38)]
    amaxes += list(gen.to_bf16((2.0 ** rng.uniform(-30, 30, 24)).astype(np.float32)).float().numpy())
    x = gen.to_bf16(_blocks_all_bf16(amaxes))
    _check(x, scale_fmt, "every bf16 value")


def _sweep_values():
    pos = oracle.e4m3.DECODE[:0x7F]
    centres = np.concatenate([(pos[:-1] + pos[1:]) / 2, pos, [448.0]]).astype(np.float32)
    offs = np.arange(-64, 65, dtype=np.int64)
    bits = centres.view(np.uint32).astype(np.int64)[:, None] + offs[None, :]
    v = bits[bits >= 0].astype(np.uint32).view(np.float32)
    v = v[np.abs(v) <= 448]
    rng = np.random.default_rng(5)
    rnd = rng.uniform(0, 448, 200_000).astype(np.float32)
    den = (rng.integers(1, 1 << 23, 2000, dtype=np.uint32)).view(np.float32)     # fp32 subnormals
    tiny = (2.0 ** rng.uniform(-40, -6, 20000)).astype(np.float32)
    vals = np.concatenate([v, rnd, den, tiny, [0.0]]).astype(np.float32)
    return np.concatenate([vals, -vals])


def test_encoder_sweep_unit_scale():
    """Blocks [448, v1..v127] have s = 1 exactly, so codes = E4M3(v) directly."""
    v = _sweep_values()
    nblk = -(-v.size // 127)
    pad = np.zeros(nblk * 127, np.float32)
    pad[:v.size] = v
    blocks = np.concatenate([np.full((nblk, 1), 448.0, np.float32), pad.reshape(nblk, 127)], 1)
    nb = nblk - nblk % 4
    x = torch.from_numpy(np.ascontiguousarray(blocks[:nb].reshape(-1, 512)))
    _check(x, None, "encoder sweep s=1")
    _check(x, "ue8m0", "encoder sweep s=1")


def test_quotient_one_ulp_above_448():
    """Maxima whose fp32 quotient amax / fl32(amax / 448) is 448 + ulp: still 0x7E."""
    rng = np.random.default_rng(9)
    cand = rng.uniform(1, 2, 400_000).astype(np.float32)
    s = (cand / np.float32(448)).astype(np.float32)
    q = (cand / s).astype(np.float32)
    hits = cand[q > 448][:4096]
    assert hits.size > 100
    rows = []
    for a in hits:
        row = np.random.default_rng(int(a.view(np.uint32))).uniform(-a, a, 128).astype(np.float32)
        row[3] = a
        row[7] = -a
        rows.append(row)
    x = torch.from_numpy(np.stack(rows).reshape(-1, 1024))
    _check(x, None, "448+ulp f32")
    hb = gen.to_bf16(np.stack(rows)).float().numpy()
    _check(gen.to_bf16(hb.reshape(-1, 1024)), None, "448+ulp bf16")


def test_zero_subclamp_and_signed_zero_blocks():
    x = np.random.default_rng(3).standard_normal((8, 1024)).astype(np.float32)
    x[0, :128] = 0.0
    x[1, 128:256] = -0.0
    x[2, 256:384] *= 1e-7
    x[3, :] = 0.0
    x[3, 5] = -0.0
    x[4, 512:640] = 9.99e-5
    for dt in ("f32", "bf16"):
        t = torch.from_numpy(x) if dt == "f32" else gen.to_bf16(x)
        _check(t, None, f"zero/clamp {dt}")
        _check(t, "ue8m0", f"zero/clamp {dt}")


def test_python_binding_matches_abi():
    from fp8_block_scaled_quant_amd import act_quant
    x = gen.activations(gen.rng_for(4), 2, 3 * 128 * 4, dtype="bf16").reshape(2, 3, 512)
    y, s = act_quant(x.to(G.device()), 128, "ue8m0")
    assert y.dtype == torch.float8_e4m3fn and y.shape == (2, 3, 512) and s.shape == (2, 3, 4)
    wq, ws = oracle.act_quant(x.float().numpy(), 128, "ue8m0")
    assert np.array_equal(y.view(torch.uint8).cpu().numpy(), wq)
    assert np.array_equal(s.cpu().numpy(), ws)
