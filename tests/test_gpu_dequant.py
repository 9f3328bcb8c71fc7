"""GPU parity for fp8_weight_dequant: output bit-identical to the oracle.

Cases: the full bandwidth workload (codes [18432, 7168], bf16 out) and its
ragged variant (18440 rows, masked edge tiles); fp32 output; every one of the
256 codes at unit scale (NaN codes must stay NaN); shapes that take the
element-wise path (column count not a multiple of 16, unaligned pointers);
scales that drive products into fp32/bf16 subnormals and past the bf16 range.
"""

import numpy as np
import pytest

import oracle
from inputs import gen
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _check(w, s, out, label, offset=0):
    G.announce(f"weight_dequant {label} shape={w.shape} out={out} offset={offset}")
    got = G.weight_dequant(w, s, out, offset=offset)
    want = oracle.weight_dequant(w, s, 128, out)
    if out == "bf16":
        g, wv = got, want
        nan = np.isnan(oracle.bf16_bits_to_f32(want))
    else:
        g, wv = got.view(np.uint32), want.view(np.uint32)
        nan = np.isnan(want)
    assert np.array_equal(np.isnan(oracle.bf16_bits_to_f32(got)) if out == "bf16" else np.isnan(got), nan)
    bad = np.argwhere((g != wv) & ~nan)
    assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[:5].tolist()}"


def test_bandwidth_workload_bf16():
    d = gen.dequant_workload()
    _check(d["w"], d["w_s"], "bf16", "workload 18432x7168")


def test_ragged_workload_bf16():
    d = gen.dequant_workload(n=18440)
    _check(d["w"], d["w_s"], "bf16", "ragged 18440x7168")


@pytest.mark.parametrize("m,n", [(256, 7168), (300, 520), (129, 1024)])
def test_fp32_output(m, n):
    d = gen.dequant_workload(m, n, seed=m + n)
    _check(d["w"], d["w_s"], "f32", "fp32 out")


def test_all_codes_unit_scale():
    w = np.tile(np.arange(256, dtype=np.uint8), (130, 4))     # [130, 1024]
    s = np.ones((2, 8), np.float32)
    _check(w, s, "f32", "all codes")
    _check(w, s, "bf16", "all codes")


@pytest.mark.parametrize("m,n", [(1, 1), (5, 7), (130, 129), (300, 500), (257, 130), (3, 4000)])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_elementwise_path_shapes(m, n, out):
    d = gen.dequant_workload(m, n, seed=m * 31 + n)
    _check(d["w"], d["w_s"], out, "odd shape")


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_unaligned_pointers(out):
    d = gen.dequant_workload(200, 256, seed=8)
    _check(d["w"], d["w_s"], out, "unaligned", offset=1)


@pytest.mark.parametrize("m,n", [(16, 16), (1, 4096), (128, 128), (131, 272)])
def test_small_vector_path(m, n):
    d = gen.dequant_workload(m, n, seed=m + 7 * n)
    _check(d["w"], d["w_s"], "bf16", "small vector")


# products past the fp32 range are inf on both sides (IEEE overflow), so numpy's
# overflow warning is the expected outcome here
@pytest.mark.filterwarnings("ignore:overflow encountered in multiply:RuntimeWarning")
def test_extreme_scales():
    w = np.tile(np.arange(256, dtype=np.uint8), (256, 2))      # [256, 512]
    w[w == 0x7F] = 0x7E
    w[w == 0xFF] = 0xFE
    s = np.array([[2.0**-133, 2.0**-126, 2.0**-100, 1.0], [2.0**100, 2.0**119, 2.0**120, 3.0e38]], np.float32)
    _check(w, s, "f32", "extreme scales")
    _check(w, s, "bf16", "extreme scales")
