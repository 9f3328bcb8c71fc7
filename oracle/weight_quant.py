"""128x128 block weight quantization (oracle; test infrastructure only).

What the pages fix (page "DeepSeek-V3 quantization_config Parameters
Explained", section "The weight_block_size Parameter: Quantization
Granularity"; page "How weight_dequant Handles Per-Block Scaling in
DeepSeek-V3 FP8 GEMM", sections "Per-Block Scaling Architecture" and "Grid
Mapping and Scale Lookup"; page "DeepSeek-V3: How Selective FP8 Stays
Stable", "Learning outcomes"):

* weights are stored as float8_e4m3fn codes split into block_size x
  block_size tiles (128 x 128 by default), each tile with one FP32 scale,
  called the inverse scale (weight_scale_inv), kept in a row-major 2-D tensor
  of shape [ceil(M / bs), ceil(N / bs)];
* dequantization multiplies a code by its tile's stored scale, y = x * s.

The pages print no formula for producing the codes and scales.  Reading taken
(R23): a tile is quantized exactly as act_quant quantizes a 1 x 128 block, with
the tile in place of the block -- amax over the tile's elements, clamped to at
least fl32(1e-4), s = fl32(amax / 448) (optionally rounded up to a power of
two, ue8m0), codes E4M3(fl32(x / s)) with RNE and saturation.  The stored
scale is s itself, so that weight_dequant's y = x * s inverts it.  Edge tiles
(M or N not a multiple of the block) take amax over their valid elements only.
"""

import numpy as np

from . import e4m3

_CLAMP = np.float32(1e-4)
_FP8_MAX = np.float32(448.0)


def _ue8m0_round_up(s: np.ndarray) -> np.ndarray:
    """Smallest power of two >= s (s > 0, finite, float32), as float32."""
    mant, exp = np.frexp(s.astype(np.float64))
    exp = np.where(mant == 0.5, exp - 1, exp)
    return np.ldexp(np.float64(1.0), exp).astype(np.float32)


def weight_quant(x: np.ndarray, block_size: int = 128, scale_fmt=None):
    """Quantize a 2-D float32 weight [M, N] per block_size x block_size tile.

    Returns ``(codes uint8 [M, N], scales float32 [ceil(M/bs), ceil(N/bs)])``.
    """
    x = np.asarray(x)
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError("weight_quant oracle takes a 2-D float32 array (bf16 widened exactly)")
    if scale_fmt not in (None, "ue8m0"):
        raise ValueError(f"unknown scale_fmt {scale_fmt!r}")
    if not np.all(np.isfinite(x)):
        raise ValueError("weight_quant oracle requires finite inputs")
    m, n = x.shape
    bs = block_size
    gm, gn = -(-m // bs), -(-n // bs)

    # Zero padding to whole tiles leaves every tile's amax unchanged (the
    # clamp keeps amax >= 1e-4 > 0); padded positions are dropped at the end.
    xp = np.zeros((gm * bs, gn * bs), dtype=np.float32)
    xp[:m, :n] = x
    tiles = xp.reshape(gm, bs, gn, bs)

    amax = np.max(np.abs(tiles), axis=(1, 3))     # [gm, gn], exact in fp32
    amax = np.maximum(amax, _CLAMP)
    s = (amax / _FP8_MAX).astype(np.float32)      # one fp32 division per tile
    if scale_fmt == "ue8m0":
        s = _ue8m0_round_up(s)

    q = (tiles / s[:, None, :, None]).astype(np.float32)   # fp32 quotient
    codes = e4m3.encode(q).reshape(gm * bs, gn * bs)[:m, :n]
    return np.ascontiguousarray(codes), s
