"""128x128 block-scaled weight dequantization (oracle; test infrastructure only).

What the pages fix (page "How weight_dequant Handles Per-Block Scaling in
DeepSeek-V3 FP8 GEMM", sections "Per-Block Scaling Architecture", "Grid Mapping
and Scale Lookup", "Dequantization Computation" and "Python Wrapper and Launch
Configuration"; page "DeepSeek-V3 quantization_config Parameters Explained",
section "The weight_block_size Parameter"):

* the weight is 2-D [M, N] (M rows, N columns) of E4M3 codes split into
  block_size x block_size tiles, 128 by default, each with its own FP32 scale
  (called weight_scale_inv) held in a row-major 2-D scale tensor;
* the scale of the tile in block-row i and block-column j sits at linear index
  i * ceil(N / block_size) + j;
* each element is converted to FP32 and multiplied by its tile's scale:
  y = x * s; edge tiles are masked.

Readings:
  R10 the scale grid is [ceil(M/bs), ceil(N/bs)] (the pages also write
      M//bs, N//bs, which agrees whenever the sizes divide).
  R11 the output is FP32 or BF16; BF16 is the FP32 product rounded to nearest
      even -- two roundings, both part of the definition.
  R12 the stored scale is multiplied, never inverted.
"""

import numpy as np

from . import e4m3


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 values (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even; NaN stays NaN."""
    v = np.asarray(v, dtype=np.float32)
    bits = v.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = (bits + 0x7FFF + lsb) >> 16
    nan = np.isnan(v)
    quiet = ((bits >> 16) | 0x0040) & 0xFFFF
    return np.where(nan, quiet, rounded).astype(np.uint16)


def weight_dequant(x: np.ndarray, s: np.ndarray, block_size: int = 128, out: str = "f32"):
    """Dequantize E4M3 codes ``x`` [M, N] with block scales ``s``.

    Returns float32 [M, N] for ``out="f32"``, or bf16 bit patterns (uint16)
    for ``out="bf16"``.
    """
    x = np.asarray(x)
    s = np.asarray(s)
    if x.ndim != 2 or x.dtype != np.uint8:
        raise ValueError("weight codes must be a 2-D uint8 array")
    if s.dtype != np.float32:
        raise TypeError("scales must be float32")
    m, n = x.shape
    gm, gn = -(-m // block_size), -(-n // block_size)
    if s.shape != (gm, gn):
        raise ValueError(f"scale grid must be {(gm, gn)}, got {s.shape}")
    if out not in ("f32", "bf16"):
        raise ValueError("out must be 'f32' or 'bf16'")

    values = e4m3.DECODE.astype(np.float32)  # every finite code is exact in fp32
    y = np.empty((m, n), dtype=np.float32)
    for i in range(gm):
        r0, r1 = i * block_size, min((i + 1) * block_size, m)
        row_scale = np.repeat(s[i], block_size)[:n]          # scale of each column's tile
        y[r0:r1] = values[x[r0:r1]] * row_scale[None, :]      # one fp32 multiply
    if out == "bf16":
        return f32_to_bf16_bits(y)
    return y
