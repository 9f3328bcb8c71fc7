"""The block GEMM at the largest operands its fast kernels address, and one row past.

The tiled kernel (m > 64) addresses A and B with 32-bit per-lane byte offsets
from the operand's base; the decode kernels with 32-bit offsets from a 64-bit
base per group of weight rows.  A product whose A or B (for m > 64) reaches
4 GiB takes the reference-structure kernel, which indexes in 64 bits.  With
K = 7168 the last size the tiled kernel takes is floor(2^32 / K) = 599,186
rows; at 599,187 rows the last row straddles byte 2^32.  These cases run, through
the C ABI:

* B of 599,186 and 599,187 rows against 80 activation rows (tiled kernel, then
  the fallback), and against 8 rows (decode kernel, B past 4 GiB);
* A of 599,186 and 599,187 rows against 256 weight rows (tiled, fallback).

Every output buffer carries canary guard bands.  Outputs are checked against
the oracle on sampled columns (B cases) or rows (A cases): the first and last,
the two around byte 2^32, both sides of a 128-row block edge, and 200 seeded
random ones.  The large operands come from the seeded chunked code generator.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_quant_amd import _lib
from inputs import gen
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

K = 7168
EDGE = (1 << 32) // K        # rows of the largest operand the tiled kernel addresses
NKB = K // 128


def _sample(n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    s = {0, 1, 127, 128, EDGE - 1, EDGE, n - 2, n - 1}
    s |= set(rng.choice(n, 200, replace=False).tolist())
    return np.array(sorted(r for r in s if 0 <= r < n))


def _big_codes(seed: int, n: int, keep: np.ndarray):
    """[n, K] E4M3 codes on the GPU, built chunk by chunk; host copies of rows `keep`."""
    dev = G.device()
    t = torch.empty((n, K), dtype=torch.uint8, device=dev)
    kept = np.empty((len(keep), K), dtype=np.uint8)
    for r0, c in gen.weight_codes_chunks(seed, n, K):
        t[r0:r0 + c.shape[0]].copy_(torch.from_numpy(c))
        sel = np.nonzero((keep >= r0) & (keep < r0 + c.shape[0]))[0]
        kept[sel] = c[keep[sel] - r0]
    torch.cuda.synchronize()
    return t, kept


def _gemm(a: torch.Tensor, a_s: torch.Tensor, b: torch.Tensor, b_s: torch.Tensor, m: int, n: int):
    """fp8_block_gemm through the C ABI into a guarded fp32 output; returns [m, n] on the GPU."""
    c = G.Guarded(m * n * 4)
    st = _lib.lib().fp8_block_gemm(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(a_s.data_ptr()),
                                   ctypes.c_void_p(b.data_ptr()), ctypes.c_void_p(b_s.data_ptr()),
                                   ctypes.c_void_p(c.ptr), _lib.F32, m, n, K, G.stream())
    assert st == _lib.OK, _lib.lib().fp8bsq_strerror(st)
    torch.cuda.synchronize()
    c.check_guards()
    return c.payload().view(torch.float32).view(m, n)


def _check(got: np.ndarray, a, a_s, b, b_s, label):
    ref = oracle.fp8_gemm(a, a_s, b, b_s)
    tol = oracle.gemm_tolerance(a, a_s, b, b_s)
    ok = oracle.gemm_check(got, ref, tol, "f32")
    assert ok.all(), f"{label}: {int((~ok).sum())} of {ok.size} sampled outputs out of the oracle bound"


@pytest.fixture(scope="module")
def big_weight():
    n = EDGE + 1
    cols = _sample(n, 1)
    G.announce(f"building weight codes [{n}, {K}] ({n * K / 2**30:.3f} GiB)")
    b, kept = _big_codes(701, n, cols)
    rng = gen.rng_for(702)
    b_s = gen.log_uniform_scales(rng, gen.scale_grid(n, K), -14, -2)
    yield b, torch.from_numpy(b_s).to(G.device()), b_s, cols, kept
    del b
    torch.cuda.empty_cache()


@pytest.mark.parametrize("m,n,kernel", [(80, EDGE, "tiled"), (80, EDGE + 1, "fallback"),
                                        (8, EDGE + 1, "decode")])
def test_weight_at_the_offset_limit(big_weight, m, n, kernel):
    b, b_s_dev, b_s, cols, kept = big_weight
    G.announce(f"max-size GEMM {m}x{n}x{K} ({kernel}): B {n * K} bytes")
    rng = gen.rng_for(710 + m)
    a = gen.weight_codes(rng, m, K)
    a_s = gen.log_uniform_scales(rng, (m, NKB), -12, -4)
    dev = G.device()
    c = _gemm(torch.from_numpy(a).to(dev), torch.from_numpy(a_s).to(dev), b[:n], b_s_dev, m, n)
    use = cols < n
    got = c[:, torch.from_numpy(cols[use]).to(dev)].cpu().numpy().astype(np.float64)
    # one weight row per sampled column, with its block's scales
    for i, j in enumerate(cols[use]):
        _check(got[:, i:i + 1], a, a_s, kept[np.nonzero(use)[0][i]][None, :], b_s[j // 128][None, :],
               f"column {j}")


@pytest.fixture(scope="module")
def big_activations():
    m = EDGE + 1
    rows = _sample(m, 2)
    G.announce(f"building activation codes [{m}, {K}] ({m * K / 2**30:.3f} GiB)")
    a, kept = _big_codes(801, m, rows)
    rng = gen.rng_for(802)
    a_s = gen.log_uniform_scales(rng, (m, NKB), -12, -4)
    yield a, torch.from_numpy(a_s).to(G.device()), a_s, rows, kept
    del a
    torch.cuda.empty_cache()


@pytest.mark.parametrize("m,kernel", [(EDGE, "tiled"), (EDGE + 1, "fallback")])
def test_activations_at_the_offset_limit(big_activations, m, kernel):
    a, a_s_dev, a_s, rows, kept = big_activations
    n = 256
    G.announce(f"max-size GEMM {m}x{n}x{K} ({kernel}): A {m * K} bytes")
    rng = gen.rng_for(810)
    b = gen.weight_codes(rng, n, K)
    b_s = gen.log_uniform_scales(rng, gen.scale_grid(n, K), -14, -2)
    dev = G.device()
    c = _gemm(a[:m], a_s_dev[:m], torch.from_numpy(b).to(dev), torch.from_numpy(b_s).to(dev), m, n)
    use = rows < m
    got = c[torch.from_numpy(rows[use]).to(dev)].cpu().numpy().astype(np.float64)
    _check(got, kept[use], a_s[rows[use]], b, b_s, f"{kernel} rows")
