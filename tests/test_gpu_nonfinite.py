"""Non-finite activations: the outputs they touch are unspecified, the rest are not.

The C ABI leaves the outputs for NaN or Inf inputs unspecified but requires the
calls to stay memory-safe.  act_quant works block by block, so a NaN or Inf
in one 1 x 128 block may change that block's codes and scale only: every other
block must still match the oracle bit for bit, and the canary bands around
every output must be untouched.  Checked for bf16 and fp32 activations, both
scale formats, and for the one-kernel act_quant_gemm path (m <= 16), whose
helper waves quantize x in every workgroup (with all of x in LDS, and through
the LDS ring at m = 12, k = 7168).
"""

import numpy as np
import pytest
import torch

import oracle
from inputs import gen
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

BAD = [float("nan"), float("inf"), float("-inf")]


def _plant(x: torch.Tensor, seed: int, count: int):
    """Put NaN / +Inf / -Inf at `count` seeded positions; returns the blocks hit."""
    rng = np.random.default_rng(seed)
    m, k = x.shape
    hit = set()
    for i in range(count):
        r, c = int(rng.integers(0, m)), int(rng.integers(0, k))
        x[r, c] = BAD[i % 3]
        hit.add((r, c // 128))
    return hit


def _clean_mask(m, k, hit):
    mask = np.ones((m, k // 128), dtype=bool)
    for r, b in hit:
        mask[r, b] = False
    return mask


def _expect(x: torch.Tensor, fmt):
    """The oracle on x with its non-finite values replaced by zero (only the
    blocks without them are compared)."""
    xf = x.float().numpy().copy()
    xf[~np.isfinite(xf)] = 0.0
    return oracle.act_quant(xf, 128, fmt)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fmt", [None, "ue8m0"])
def test_act_quant_confines_non_finite_blocks(dtype, fmt):
    m, k = 300, 1024
    x = gen.activations(gen.rng_for(91), m, k, dtype=dtype)
    hit = _plant(x, 92, 40)
    G.announce(f"act_quant {dtype} fmt={fmt} with {len(hit)} non-finite blocks")
    codes, scales = G.act_quant(x.to(G.device()), fmt)     # checks the canary bands
    wq, ws = _expect(x, fmt)
    clean = _clean_mask(m, k, hit)
    assert np.array_equal(scales.view(np.uint32)[clean], ws.view(np.uint32)[clean])
    cb = np.repeat(clean, 128, axis=1)
    assert np.array_equal(codes[cb], wq[cb])


@pytest.mark.parametrize("m,k", [(1, 2048), (5, 2048), (16, 2048), (12, 7168)])
def test_fused_act_quant_gemm_confines_non_finite_blocks(m, k):
    d = gen.custom_gemm(seed=93 + m, m=m, n=700, k=k)
    x = d["x"]
    hit = _plant(x, 94 + m, 3)
    G.announce(f"act_quant_gemm m={m} k={k} with {len(hit)} non-finite blocks")
    _, codes, scales = G.act_quant_gemm(x.to(G.device()), d["w"], d["w_s"], None, "bf16")
    wq, ws = _expect(x, None)
    clean = _clean_mask(m, k, hit)
    assert np.array_equal(scales.view(np.uint32)[clean], ws.view(np.uint32)[clean])
    cb = np.repeat(clean, 128, axis=1)
    assert np.array_equal(codes[cb], wq[cb])
