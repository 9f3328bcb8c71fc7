"""Pins for the oracle's block-scaled GEMM and its error bound.

* exact rational brute force on tiny problems (Python ``fractions``);
* agreement with dequantize-then-multiply (A_hat @ B_hat^T in float64);
* one K block: C = a_s * b_s * P exactly, P from integer arithmetic;
* unit scales and small integer code values: equals the int64 product A B^T;
* homogeneity pins the scale indexing: doubling one row of a_s doubles one
  row of C, doubling one block-row of b_s doubles exactly those 128 columns,
  zeroing one K-block's scales removes exactly that block;
* the bound: 1e-3 * sum_k |a_k b_k| checked against brute force.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from inputs import gen
from tests.exact import torch_e4m3_table

TABLE = torch_e4m3_table()


def _problem(seed, m, n, k, lo=-12, hi=-4):
    rng = np.random.default_rng(seed)
    a = gen.weight_codes(rng, m, k)
    a_s = gen.log_uniform_scales(rng, (m, k // 128), -8, 0)
    b = gen.weight_codes(rng, n, k)
    b_s = gen.log_uniform_scales(rng, gen.scale_grid(n, k), lo, hi)
    return a, a_s, b, b_s


def exact_gemm(a, a_s, b, b_s):
    m, k = a.shape
    n = b.shape[0]
    out = [[Fraction(0)] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            tot = Fraction(0)
            for kb in range(k // 128):
                p = sum(Fraction(float(TABLE[a[i, kk]])) * Fraction(float(TABLE[b[j, kk]]))
                        for kk in range(kb * 128, kb * 128 + 128))
                tot += p * Fraction(float(a_s[i, kb])) * Fraction(float(b_s[j // 128, kb]))
            out[i][j] = tot
    return out


def check_exact(fp8_gemm, seed, m, n, k):
    a, a_s, b, b_s = _problem(seed, m, n, k)
    c = fp8_gemm(a, a_s, b, b_s)
    ex = exact_gemm(a, a_s, b, b_s)
    nkb = k // 128
    for i in range(m):
        for j in range(n):
            mag = sum(abs(Fraction(float(TABLE[a[i, kk]])) * Fraction(float(TABLE[b[j, kk]])))
                      * Fraction(float(a_s[i, kk // 128])) * Fraction(float(b_s[j // 128, kk // 128]))
                      for kk in range(k))
            assert abs(Fraction(float(c[i, j])) - ex[i][j]) <= 4 * nkb * Fraction(1, 2**53) * mag


@pytest.mark.parametrize("seed,m,n,k", [(0, 2, 3, 128), (1, 3, 2, 256), (2, 4, 4, 384)])
def test_exact_bruteforce(seed, m, n, k):
    check_exact(oracle.fp8_gemm, seed, m, n, k)


def test_exact_bruteforce_second_weight_block():
    a, a_s, b, b_s = _problem(5, 2, 130, 256)
    c = oracle.fp8_gemm(a, a_s, b, b_s)
    for j in (0, 127, 128, 129):
        bj = b[j:j + 1]
        bsj = b_s[j // 128:j // 128 + 1]
        ex = exact_gemm(a, a_s, bj, bsj)
        for i in range(2):
            assert abs(Fraction(float(c[i, j])) - ex[i][0]) <= abs(ex[i][0]) * Fraction(1, 2**48)


def check_vs_dequant_matmul(fp8_gemm, seed, m, n, k):
    a, a_s, b, b_s = _problem(seed, m, n, k)
    c = fp8_gemm(a, a_s, b, b_s)
    a_hat = TABLE[a] * np.repeat(a_s.astype(np.float64), 128, 1)
    b_full = np.repeat(np.repeat(b_s.astype(np.float64), 128, 0)[:n], 128, 1)
    b_hat = TABLE[b] * b_full
    ref = a_hat @ b_hat.T
    mag = np.abs(a_hat) @ np.abs(b_hat).T
    assert np.all(np.abs(c - ref) <= 1e-12 * mag)


@pytest.mark.parametrize("seed,m,n,k", [(10, 16, 256, 512), (11, 33, 300, 1024), (12, 1, 129, 128)])
def test_vs_dequant_matmul(seed, m, n, k):
    check_vs_dequant_matmul(oracle.fp8_gemm, seed, m, n, k)


def check_single_block(fp8_gemm):
    a, a_s, b, b_s = _problem(20, 8, 200, 128)
    c = fp8_gemm(a, a_s, b, b_s)
    ia = (TABLE[a] * 2**9).astype(np.int64)          # E4M3 values are multiples of 2^-9
    ib = (TABLE[b] * 2**9).astype(np.int64)
    p = (ia @ ib.T).astype(np.float64) * 2.0**-18    # exact
    scale = a_s[:, 0].astype(np.float64)[:, None] * b_s[np.arange(200) // 128, 0].astype(np.float64)[None, :]
    assert np.array_equal(c, p * scale)


def test_single_block_exact():
    check_single_block(oracle.fp8_gemm)


def check_integer_codes(fp8_gemm):
    rng = np.random.default_rng(30)
    ints = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48, 5: 0x4A, 6: 0x4C, 7: 0x4E, 8: 0x50}
    vals = rng.integers(-8, 9, size=(7, 384))
    valsb = rng.integers(-8, 9, size=(140, 384))
    enc = np.vectorize(lambda v: ints[abs(v)] | (0x80 if v < 0 else 0))
    a, b = enc(vals).astype(np.uint8), enc(valsb).astype(np.uint8)
    assert np.array_equal(TABLE[a], vals) and np.array_equal(TABLE[b], valsb)
    c = fp8_gemm(a, np.ones((7, 3), np.float32), b, np.ones((2, 3), np.float32))
    assert np.array_equal(c, (vals @ valsb.T).astype(np.float64))


def test_integer_codes():
    check_integer_codes(oracle.fp8_gemm)


def check_homogeneity(fp8_gemm):
    a, a_s, b, b_s = _problem(40, 6, 300, 384)
    c = fp8_gemm(a, a_s, b, b_s)
    a2 = a_s.copy()
    a2[3] *= 2
    c2 = fp8_gemm(a, a2, b, b_s)
    assert np.array_equal(c2[3], 2 * c[3]) and np.array_equal(np.delete(c2, 3, 0), np.delete(c, 3, 0))
    b2 = b_s.copy()
    b2[1] *= 2
    c3 = fp8_gemm(a, a_s, b, b2)
    assert np.array_equal(c3[:, 128:256], 2 * c[:, 128:256])
    assert np.array_equal(c3[:, :128], c[:, :128]) and np.array_equal(c3[:, 256:], c[:, 256:])
    a4 = a_s.copy()
    a4[:, 1] = 0
    c4 = fp8_gemm(a, a4, b, b_s)
    keep = np.r_[0:128, 256:384]
    ref = fp8_gemm(np.ascontiguousarray(a[:, keep]), np.ascontiguousarray(a_s[:, [0, 2]]),
                   np.ascontiguousarray(b[:, keep]), np.ascontiguousarray(b_s[:, [0, 2]]))
    assert np.allclose(c4, ref, rtol=1e-15, atol=0)
    rows = np.array([5, 0, 2])
    assert np.array_equal(fp8_gemm(a, a_s, b, b_s, rows=rows), c[rows])


def test_homogeneity_and_indexing():
    check_homogeneity(oracle.fp8_gemm)


def test_tolerance_bruteforce():
    a, a_s, b, b_s = _problem(50, 3, 5, 256)
    t = oracle.gemm_tolerance(a, a_s, b, b_s)
    for i in range(3):
        for j in range(5):
            mag = sum(abs(float(TABLE[a[i, kk]]) * float(TABLE[b[j, kk]]))
                      * float(a_s[i, kk // 128]) * float(b_s[j // 128, kk // 128]) for kk in range(256))
            assert abs(t[i, j] - 1e-3 * mag) <= 1e-12 * mag
    c = oracle.fp8_gemm(a, a_s, b, b_s)
    assert np.all(np.abs(c) <= t * 1e3 * (1 + 1e-12))
    good = oracle.gemm_check(c + 0.5 * t, c, t, "f32")
    bad = oracle.gemm_check(c + 2.0 * t + 1e-30, c, t, "f32")
    assert good.all() and not bad.any()
    assert not oracle.gemm_check(np.full_like(c, np.nan), c, t).any()
