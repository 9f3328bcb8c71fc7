"""fp8_block_gemm_split_noalloc (the split-K product with the library's static
per-GPU scratch instead of a caller's workspace) against fp8_block_gemm_split
with a workspace, through the C ABI.

Both run the same kernels in the same summation order, so outputs must be
bit-identical; the split rows are also held to the oracle bound.  Two calls in
a row reuse the scratch, the second on a smaller problem, then a shape that
does not split, and scale_fmt ue8m0 (with its guard) on the split path.
"""

import ctypes

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as fb
import oracle
from fp8_block_scaled_quant_amd import _lib
from inputs import gen
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _noalloc(a_dev, a_s_dev, b, b_s, out, ue8m0=False):
    dev = G.device()
    m, k = a_dev.shape
    n = b.shape[0]
    bd = torch.from_numpy(b).to(dev)
    bsd = torch.from_numpy(b_s).to(dev)
    esz = 2 if out == "bf16" else 4
    c = G.Guarded(m * n * esz)
    st = _lib.lib().fp8_block_gemm_split_noalloc(
        ctypes.c_void_p(a_dev.data_ptr()), ctypes.c_void_p(a_s_dev.data_ptr()),
        ctypes.c_void_p(bd.data_ptr()), ctypes.c_void_p(bsd.data_ptr()), ctypes.c_void_p(c.ptr),
        _lib.BF16 if out == "bf16" else _lib.F32, m, n, k,
        _lib.SCALE_UE8M0 if ue8m0 else _lib.SCALE_NONE, G.stream())
    assert st == _lib.OK, st
    torch.cuda.synchronize()
    c.check_guards()
    raw = c.payload().cpu().numpy()
    if out == "bf16":
        return ((raw.view(np.uint16).reshape(m, n).astype(np.uint32) << 16).view(np.float32)).astype(np.float64)
    return raw.view(np.float32).reshape(m, n).astype(np.float64)


def _case(seed, m, n, k, fmt=None):
    d = gen.custom_gemm(seed=seed, m=m, n=n, k=k, outliers=True)
    a, a_s = fb.act_quant(d["x"].to(G.device()), 128, fmt)
    return a.view(torch.uint8), a_s, d["w"], d["w_s"]


def _check(m, n, k, seed, out, fmt=None):
    lib = _lib.lib()
    need = lib.fp8_block_gemm_split_workspace(m, n, k)
    assert need <= _lib.SPLIT_SCRATCH_BYTES
    a, a_s, w, ws = _case(seed, m, n, k, fmt)
    G.announce(f"split_noalloc m={m} n={n} k={k} {out} scale_fmt={fmt} (workspace {need} B)")
    got = _noalloc(a, a_s, w, ws, out, ue8m0=fmt == "ue8m0")
    want, _ = G.block_gemm_split(a, a_s, w, ws, out, ue8m0=fmt == "ue8m0")
    assert np.array_equal(got.view(np.uint64), want.view(np.uint64)), \
        f"{int((got != want).sum())} outputs differ from fp8_block_gemm_split"
    an, asn = a.cpu().numpy(), a_s.cpu().numpy()
    rows = np.unique(np.concatenate([[0, m - 1], np.random.default_rng(seed).choice(m, 64, replace=False)]))
    c = oracle.fp8_gemm(an, asn, w, ws, rows=rows)
    tol = oracle.gemm_tolerance(an, asn, w, ws, rows=rows)
    assert oracle.gemm_check(got[rows], c, tol, out).all()
    return need


def test_two_calls_in_a_row_then_smaller():
    # 272 tiles of 256 x 256 = one full round + 16 split in 4 parts; then 8 tiles, no full round
    first = _check(4096, 4352, 8192, seed=71, out="bf16")
    second = _check(512, 1024, 8192, seed=72, out="f32")
    assert first > second > 0


def test_no_split_shape_and_ue8m0():
    lib = _lib.lib()
    assert lib.fp8_block_gemm_split_workspace(300, 512, 1024) == 0
    _check(300, 512, 1024, seed=73, out="bf16")
    _check(512, 1024, 8192, seed=74, out="bf16", fmt="ue8m0")
