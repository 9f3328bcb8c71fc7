"""Dynamic 1x128 activation quantization (oracle; test infrastructure only).

What the pages fix (page "Understanding Dynamic and Static Activation
Quantization Schemes in DeepSeek-V3", section "How Dynamic Activation
Quantization Works"; page "DeepSeek-V3 quantization_config Parameters
Explained", section "The activation_scheme Parameter: Runtime Scaling
Strategy" and its FAQ):

* the input is contiguous and its last dimension is a multiple of the block
  size, 128 by default; every 1 x block_size run along the last dimension is a
  block with its own scale, computed at run time from the block's values;
* amax is the block's largest magnitude, clamped to at least 1e-4;
* s = amax / 448, 448 being the largest E4M3 value;
* scale_fmt "ue8m0" optionally rounds s to a power of two;
* outputs are float8_e4m3fn codes with x's shape and one FP32 scale per block.

The pages dequantize by multiplying codes by the scale (same page, section "How
Static Activation Quantization Differs"), so quantizing divides by it.

Readings taken where the pages are silent:
  R1  q = E4M3(fl32(x / s)): one IEEE fp32 division, then E4M3 RNE.  Both
      roundings are part of the definition (neither x * fl32(1/s) nor the exact
      quotient rounded once is meant).
  R2  s = fl32(amax / 448): one correctly rounded fp32 division.
  R3  the clamp is fl32(1e-4) and comes before the division and before ue8m0.
  R4  ue8m0 rounds UP to the smallest power of two >= fl32(amax/448), so no
      |x / s| exceeds 448; it is taken from the bits (frexp), never from a
      rounded log2.  The scale stays FP32.
  R5-R8  as in ``oracle.e4m3``: RNE, saturation, signed zero kept.
  R7  inputs must be finite; a NaN or Inf raises.
  R18 an N-D input is treated as [numel / K, K]; scales keep x's leading shape.
"""

import numpy as np

from . import e4m3

_CLAMP = np.float32(1e-4)
_FP8_MAX = np.float32(448.0)


def _ue8m0_round_up(s: np.ndarray) -> np.ndarray:
    """Smallest power of two >= s (s > 0, finite, float32), as float32."""
    mant, exp = np.frexp(s.astype(np.float64))  # s = mant * 2^exp, mant in [0.5, 1)
    exp = np.where(mant == 0.5, exp - 1, exp)
    return np.ldexp(np.float64(1.0), exp).astype(np.float32)


def act_quant(x: np.ndarray, block_size: int = 128, scale_fmt=None):
    """Quantize ``x`` (float32 values; bf16 inputs widened exactly) per 1 x block.

    Returns ``(codes uint8 x.shape, scales float32 x.shape[:-1] + (K/block,))``.
    """
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("act_quant oracle takes float32 values (bf16 widened exactly)")
    if scale_fmt not in (None, "ue8m0"):
        raise ValueError(f"unknown scale_fmt {scale_fmt!r}")
    if x.ndim < 1 or x.shape[-1] % block_size != 0:
        raise ValueError("last dimension must be a multiple of block_size")
    if not np.all(np.isfinite(x)):
        raise ValueError("act_quant oracle requires finite inputs")
    k = x.shape[-1]
    nb = k // block_size
    xb = x.reshape(-1, nb, block_size)

    amax = np.max(np.abs(xb), axis=-1)            # exact in fp32
    amax = np.maximum(amax, _CLAMP)               # R3
    s = (amax / _FP8_MAX).astype(np.float32)      # R2: fp32 division
    if scale_fmt == "ue8m0":
        s = _ue8m0_round_up(s)                    # R4

    q = (xb / s[:, :, None]).astype(np.float32)   # R1: fp32 quotient
    codes = e4m3.encode(q)                        # R1, R5-R8: E4M3 RNE

    return codes.reshape(x.shape), s.reshape(x.shape[:-1] + (nb,))
