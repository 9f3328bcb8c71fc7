"""Exact-arithmetic helpers for the oracle pins (no code shared with ``oracle/``).

Rational arithmetic (``fractions.Fraction``) gives reference values that do not
depend on numpy's or the oracle's floating point; the E4M3 value table used here
comes from torch's own CPU float8_e4m3fn decode, not from the oracle.
"""

from fractions import Fraction

import numpy as np
import torch


def f32_round(q: Fraction) -> np.float32:
    """Round a rational to the nearest binary32 value, ties to even (with subnormals)."""
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    quantum = Fraction(2) ** (max(e, -126) - 23)
    k = a / quantum
    n = k.numerator // k.denominator
    rem = k - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * quantum
    if val >= Fraction(2) ** 128:
        return np.float32(sign * np.inf)
    return np.float32(sign * float(val))


def frac(v) -> Fraction:
    return Fraction(float(v))


def torch_e4m3_table() -> np.ndarray:
    """float64 value of every code, decoded by torch's CPU float8_e4m3fn."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def nearest_e4m3_bruteforce(v: float, table: np.ndarray) -> int:
    """Code of the finite E4M3 value nearest to v; ties go to the even code;
    magnitudes >= 448 saturate.  Sign of zero follows v.  Scans every code."""
    fv = Fraction(float(v))
    neg = fv < 0 or (fv == 0 and np.signbit(v))
    a = abs(fv)
    best, best_d = None, None
    for c in range(0x7F):                       # non-negative finite codes
        d = abs(a - Fraction(float(table[c])))
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    if a >= 448:
        best = 0x7E
    return best | (0x80 if neg else 0)
