"""GPU parity for fp8_weight_quant: codes and scales bit-identical to the oracle.

Cases: the full weight workload [18432, 7168] bf16 (both scale formats) and
its ragged variant [18440, 7168]; fp32 input; shapes with edge tiles on the
vectorized path (n % 8 == 0) and on the element-wise path (n % 8 != 0,
unaligned pointers); an all-zero tile and negative zeros; the quantize ->
dequantize round trip through the GPU dequantizer; and the Python binding.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as fb
import oracle
from inputs import gen
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _check(w: torch.Tensor, scale_fmt, label, offset=0):
    G.announce(f"weight_quant {label} shape={tuple(w.shape)} dtype={w.dtype} fmt={scale_fmt} offset={offset}")
    q, s = G.weight_quant(w.to(G.device()), scale_fmt, offset=offset)
    wq, ws = oracle.weight_quant(w.float().numpy(), 128, scale_fmt)
    assert np.array_equal(s.view(np.uint32), ws.view(np.uint32)), \
        f"{int((s.view(np.uint32) != ws.view(np.uint32)).sum())} scales differ"
    bad = np.argwhere(q != wq)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:5].tolist()}"
    return q, s


@pytest.mark.parametrize("scale_fmt", [None, "ue8m0"])
def test_weight_workload(scale_fmt):
    _check(gen.weight_quant_workload()["w"], scale_fmt, "workload 18432x7168")


def test_ragged_workload():
    _check(gen.weight_quant_workload(n=18440)["w"], None, "ragged 18440x7168")


@pytest.mark.parametrize("m,n", [(256, 7168), (300, 520), (130, 200), (1, 8)])
@pytest.mark.parametrize("scale_fmt", [None, "ue8m0"])
def test_fp32_input(m, n, scale_fmt):
    _check(gen.weight_quant_workload(m, n, seed=m + n, dtype="f32")["w"], scale_fmt, "fp32 in")


@pytest.mark.parametrize("m,n", [(129, 136), (384, 640), (1, 128), (200, 8)])
def test_vector_path_edge_tiles(m, n):
    _check(gen.weight_quant_workload(m, n, seed=3 * m + n)["w"], None, "edge tiles")


@pytest.mark.parametrize("m,n", [(1, 1), (5, 7), (130, 129), (257, 130 + 3), (3, 4001)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_elementwise_path_shapes(m, n, dtype):
    _check(gen.weight_quant_workload(m, n, seed=m * n, dtype=dtype)["w"], None, "element-wise")


def test_unaligned_pointers_take_elementwise_path():
    w = gen.weight_quant_workload(256, 512, seed=77)["w"]
    _check(w, None, "unaligned", offset=1)
    _check(w, "ue8m0", "unaligned", offset=3)


def test_zero_tile_and_negative_zero():
    w = torch.randn(256, 384).to(torch.bfloat16)
    w[128:, 128:256] = 0.0
    w[130, 130] = -0.0
    w[0, 0] = -0.0
    q, s = _check(w, None, "zero tile")
    assert s[1, 1].view(np.uint32) == 0x346FACAD
    assert q[130, 130] == 0x80 and q[0, 0] == 0x80 and q[131, 131] == 0x00


def test_round_trip_through_gpu_dequant():
    w = gen.weight_quant_workload(1024, 2048, seed=9)["w"]
    G.announce("weight_quant -> weight_dequant round trip 1024x2048")
    dev = G.device()
    y, s = fb.weight_quant(w.to(dev))
    back = fb.weight_dequant(y, s, 128, torch.float32).cpu().double().numpy()
    x = w.float().double().numpy()
    srep = np.repeat(np.repeat(s.cpu().double().numpy(), 128, 0), 128, 1)
    t = np.abs(x / srep)
    ulp = oracle.e4m3.ulp(t)
    assert np.all(np.abs(back - x) <= (ulp / 2 + t * 2.0**-23) * srep + np.abs(back) * 2.0**-24)


def test_python_binding_matches_c_abi():
    w = gen.weight_quant_workload(384, 768, seed=5)["w"]
    G.announce("weight_quant binding 384x768")
    y, s = fb.weight_quant(w.to(G.device()), 128, "ue8m0")
    q, sc = G.weight_quant(w.to(G.device()), "ue8m0")
    assert y.dtype == torch.float8_e4m3fn and tuple(s.shape) == (3, 6)
    assert np.array_equal(y.view(torch.uint8).cpu().numpy(), q)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), sc.view(np.uint32))
    with pytest.raises(ValueError):
        fb.weight_quant(w)                      # CPU tensor: no fallback
