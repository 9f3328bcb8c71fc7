"""Pins for the oracle's bf16 helpers and the BF16 half of the GEMM bound.

The GEMM's BF16 outputs are held to |gpu - C| <= T + ulp_bf16(C), where T is
1e-3 * sum_k |a_k b_k| and ulp_bf16(C) is one bf16 ulp at the magnitude of the
oracle value C (page "DeepSeek-V3: How Selective FP8 Stays Stable", section
"Lower precision is a constrained budget": outputs may be BF16).  What fixes
each piece here, independently of the oracle:

* ``bf16_ulp``: the spacing of adjacent bf16 values, taken from torch's own
  bf16 -> float64 decode of every finite bit pattern, at each bf16 value, at
  the midpoint of each gap and just below each next value (where a rounded
  log2 slips into the wrong binade); zero and the subnormal floor (2^-133);
  sign symmetry;
* ``gemm_check(out="bf16")``: exact-rational brute force on small GEMMs built
  so that every product is non-negative (then T is 1e-3 * C and the ulp term
  matters), with errors placed just inside and just outside T + ulp; values
  just below a power of two whose GPU value lies above it (the ulp must be
  taken at C, not at the GPU value); NaN and Inf rejected;
* ``bf16_bits_to_f32``: all 65,536 bit patterns against torch's bf16 -> fp32.
"""

import importlib
from fractions import Fraction

import numpy as np
import torch

import oracle
from tests.exact import torch_e4m3_table

gemm_mod = importlib.import_module("oracle.fp8_gemm")

TABLE = torch_e4m3_table()


def torch_bf16_values(bits: np.ndarray) -> np.ndarray:
    """float64 value of each bf16 bit pattern, decoded by torch."""
    t = torch.from_numpy(np.asarray(bits, dtype=np.int64)).to(torch.int32).to(torch.int16)
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def exact_bf16_ulp(q: Fraction) -> Fraction:
    """Spacing of bf16 values in the binade of |q| (2^-133 below 2^-126), exactly."""
    a = abs(q)
    if a == 0:
        return Fraction(1, 2**133)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    return Fraction(2) ** (max(e, -126) - 7)


# ----------------------------------------------------------------- bf16_ulp

def check_ulp_spacing(bf16_ulp):
    bits = np.arange(0x0000, 0x7F80)                 # every finite non-negative pattern
    v = torch_bf16_values(bits)
    nxt = torch_bf16_values(np.append(bits[1:], 0x7F80))
    nxt[-1] = v[-1] + (v[-1] - v[-2])                 # past the largest finite value: same binade
    gap = nxt - v                                     # exact: both are bf16 values
    assert np.array_equal(bf16_ulp(v), gap), "ulp at bf16 values"
    assert np.array_equal(bf16_ulp(-v), gap), "ulp is symmetric in the sign"
    assert np.array_equal(bf16_ulp(v + gap / 2), gap), "ulp inside a gap"
    below = np.nextafter(nxt, 0.0)                    # just below the next bf16 value
    assert np.array_equal(bf16_ulp(below), gap), "ulp just below the next value"


def check_ulp_special(bf16_ulp):
    assert bf16_ulp(np.array([0.0]))[0] == 2.0**-133
    assert bf16_ulp(np.array([-0.0]))[0] == 2.0**-133
    for k in range(-140, 130):
        p = 2.0**k
        assert bf16_ulp(np.array([p]))[0] == 2.0 ** (max(k, -126) - 7), k
        assert bf16_ulp(np.array([np.nextafter(p, 0.0)]))[0] == 2.0 ** (max(k - 1, -126) - 7), k


def test_bf16_ulp_spacing():
    check_ulp_spacing(gemm_mod.bf16_ulp)


def test_bf16_ulp_special_values():
    check_ulp_special(gemm_mod.bf16_ulp)


# ------------------------------------------------------- gemm_check(out="bf16")

def _positive_problem(seed, m, n, k, lo_code=0x20, hi_code=0x5F):
    """Codes with non-negative values only, and assorted scales: no cancellation,
    so sum_k |a_k b_k| = C and the ulp term is a fixed share of the bound."""
    rng = np.random.default_rng(seed)
    a = rng.integers(lo_code, hi_code, size=(m, k)).astype(np.uint8)
    b = rng.integers(lo_code, hi_code, size=(n, k)).astype(np.uint8)
    a_s = (2.0 ** rng.uniform(-30, 30, size=(m, k // 128))).astype(np.float32)
    b_s = (2.0 ** rng.uniform(-30, 30, size=(-(-n // 128), k // 128))).astype(np.float32)
    return a, a_s, b, b_s


def _exact(a, a_s, b, b_s):
    m, k = a.shape
    n = b.shape[0]
    c = [[Fraction(0)] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            tot = Fraction(0)
            for kk in range(k):
                tot += (Fraction(float(TABLE[a[i, kk]])) * Fraction(float(TABLE[b[j, kk]]))
                        * Fraction(float(a_s[i, kk // 128])) * Fraction(float(b_s[j // 128, kk // 128])))
            c[i][j] = tot
    return c


def check_gemm_bound_bf16(gemm_check, seed=0, m=3, n=5, k=256):
    a, a_s, b, b_s = _positive_problem(seed, m, n, k)
    c = oracle.fp8_gemm(a, a_s, b, b_s)
    tol = oracle.gemm_tolerance(a, a_s, b, b_s)
    ex = _exact(a, a_s, b, b_s)
    for sign in (1, -1):
        inside = np.empty((m, n))
        outside = np.empty((m, n))
        for i in range(m):
            for j in range(n):
                bound = Fraction(1, 1000) * ex[i][j] + exact_bf16_ulp(ex[i][j])   # sum |ab| = C here
                inside[i, j] = float(ex[i][j] + sign * bound * Fraction(999, 1000))
                outside[i, j] = float(ex[i][j] + sign * bound * Fraction(1001, 1000))
        assert gemm_check(inside, c, tol, "bf16").all(), "error just inside T + ulp rejected"
        assert not gemm_check(outside, c, tol, "bf16").any(), "error just outside T + ulp accepted"
    # an error of T + 0.6 ulp: inside the BF16 bound, outside the FP32 one
    half = np.empty((m, n))
    for i in range(m):
        for j in range(n):
            half[i, j] = float(ex[i][j] * Fraction(1001, 1000) + exact_bf16_ulp(ex[i][j]) * Fraction(6, 10))
    assert gemm_check(half, c, tol, "bf16").all()
    assert not gemm_check(half, c, tol, "f32").any()


def check_ulp_taken_at_c(gemm_check):
    """C just below a power of two with the GPU value above it: the bound's ulp is
    C's (half of the GPU value's)."""
    # K = 128, every A code 1.0, row j of B: 127 codes of 2.0 and one 1.0 -> C = 255 * s
    one, two = 0x38, 0x40
    a = np.full((2, 128), one, np.uint8)
    b = np.full((3, 128), two, np.uint8)
    b[:, 0] = one
    assert TABLE[one] == 1.0 and TABLE[two] == 2.0
    for s in (1.0, 2.0**-20, 2.0**40):
        a_s = np.full((2, 1), s, np.float32)
        b_s = np.ones((1, 1), np.float32)
        c = oracle.fp8_gemm(a, a_s, b, b_s)
        tol = oracle.gemm_tolerance(a, a_s, b, b_s)
        cv = 255.0 * s
        assert np.all(c == cv) and np.allclose(tol, 1e-3 * cv, rtol=1e-15)
        u = s            # bf16 spacing in [128 s, 256 s)
        gpu = np.full_like(c, cv + 1e-3 * cv + 1.5 * u)     # above 256 s, where the spacing is 2 s
        assert np.all(gpu > 256.0 * s)
        assert not gemm_check(gpu, c, tol, "bf16").any(), "ulp taken at the GPU value"
        gpu = np.full_like(c, cv + 1e-3 * cv + 0.9 * u)
        assert gemm_check(gpu, c, tol, "bf16").all()


def check_nonfinite_rejected(gemm_check):
    c = np.array([[1.0, -2.0, 0.0]])
    tol = np.array([[1.0, 1.0, 1.0]])
    for bad in (np.nan, np.inf, -np.inf):
        assert not gemm_check(np.full_like(c, bad), c, tol, "bf16").any()


def test_gemm_check_bf16_bruteforce():
    check_gemm_bound_bf16(oracle.gemm_check)
    check_gemm_bound_bf16(oracle.gemm_check, seed=1, m=2, n=130, k=384)


def test_gemm_check_ulp_at_oracle_value():
    check_ulp_taken_at_c(oracle.gemm_check)


def test_gemm_check_nonfinite():
    check_nonfinite_rejected(oracle.gemm_check)


# ----------------------------------------------------------- bf16_bits_to_f32

def check_bits_to_f32(bits_to_f32):
    bits = np.arange(65536, dtype=np.int64)
    got = bits_to_f32(bits.astype(np.uint16))
    assert got.dtype == np.float32
    t = torch.from_numpy(bits).to(torch.int32).to(torch.int16).view(torch.bfloat16).to(torch.float32).numpy()
    nan = np.isnan(t)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), t[~nan].view(np.uint32))


def test_bf16_bits_to_f32_exhaustive():
    check_bits_to_f32(oracle.bf16_bits_to_f32)
