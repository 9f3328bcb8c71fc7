"""E4M3FN code table and encoder (oracle; test infrastructure only).

Format, as the pages give it: "e4m3" maps to ``torch.float8_e4m3fn`` -- 4
exponent bits, 3 mantissa bits, the "FN" (finite) variant with no infinities
(page "DeepSeek-V3 quantization_config Parameters Explained", section "The fmt
Parameter: FP8 Storage Format (e4m3)"; page "Understanding Dynamic and Static
Activation Quantization Schemes in DeepSeek-V3", FAQ "Why does DeepSeek-V3 use
FP8 E4M3FN ..."), and 448 is its largest representable value (quantization_config
page, section "The activation_scheme Parameter").

The field layout below is the standard definition of that format: sign bit,
4-bit exponent with bias 7, 3-bit mantissa; exponent field 0 holds the
subnormals m/8 * 2^-6; the single all-ones pattern (exponent 15, mantissa 7)
is NaN in each sign; everything else is finite.

Readings (the pages give no rounding rule for the encoder):
  * round to nearest, ties to the even code (mantissa LSB 0);
  * magnitudes at or above 448 saturate to +-448 (no overflow to NaN);
  * the sign is kept on zero: a negative value that rounds to zero gives 0x80;
  * NaN encodes to 0x7F.
"""

import numpy as np

NAN_CODE = 0x7F
MAX_FINITE = 448.0


def _decode_one(code: int) -> float:
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


#: float64 value of every one of the 256 codes (NaN at 0x7F and 0xFF).
DECODE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)
DECODE.setflags(write=False)

# Non-negative finite values in code order: codes 0x00..0x7E are monotonic.
_POS = DECODE[:0x7F].copy()
assert np.all(np.diff(_POS) > 0) and _POS[-1] == MAX_FINITE


def decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes (uint8, any shape) -> float64 values (exact)."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("E4M3 codes must be uint8")
    return DECODE[codes]


def encode(v: np.ndarray) -> np.ndarray:
    """fp32 (or any float) values -> E4M3 codes, RNE with saturation.

    Every comparison is exact in float64: the table values and the midpoints
    between neighbours are dyadic with at most 5 significant bits, and a
    float32 input converts to float64 exactly.
    """
    v = np.asarray(v)
    a = np.abs(v.astype(np.float64))
    sign = np.signbit(v)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    # index of the largest table value <= a (a >= 0, so idx >= 0)
    idx = np.searchsorted(_POS, a, side="right") - 1
    idx = np.clip(idx, 0, 0x7E)
    nxt = np.minimum(idx + 1, 0x7E)
    lo = _POS[idx]
    hi = _POS[nxt]
    mid = (lo + hi) * 0.5
    round_up = (a > mid) | ((a == mid) & ((idx & 1) == 1))
    code = np.where(round_up, nxt, idx)
    code = np.where(a >= MAX_FINITE, 0x7E, code)
    code = code | (sign.astype(np.int64) << 7)
    code = np.where(nan, NAN_CODE, code)
    return code.astype(np.uint8)


def ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of E4M3 values at magnitude |v| (2^-9 in the subnormal range)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(np.where(a > 0, e, -6.0), -6.0)
    return np.ldexp(1.0, (e - 3).astype(np.int64))
