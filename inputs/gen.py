"""Seeded input generators for the five workloads.

Recipe (one ``numpy.random.default_rng(seed)`` stream per workload; draws in
the order activations, then weight codes, then weight scales):

* activations: ``standard_normal`` fp32; optionally 0.1% of the elements
  (exactly round(0.001 * numel) distinct positions, chosen uniformly) are
  multiplied by 100 in fp32; optionally one 1x128 block per 128-row group is
  zeroed (row 128*g + U[0,128), block U[0, K/128)); then cast to bf16 (round to
  nearest even, torch's CPU cast) when the workload is bf16.
* weight codes: uniform over the 254 finite E4M3 codes (0x7F and 0xFF, the two
  NaNs, excluded; +-0 and subnormals included).
* block scales: float32(2 ** U[lo, hi]) (log-uniform).
* weights to quantize: ``standard_normal`` fp32 times a per-128x128-tile
  magnitude 2 ** U[-10, 0]; 0.01% of the elements multiplied by 100; one
  all-zero tile in every 8th row of tiles (tile column U[0, ceil(K/128)));
  then cast to bf16.

Operands of 4 GiB and more (the size-limit tests) come in chunks:
``weight_codes_chunks`` draws the weight-code distribution chunk by chunk from
one generator, and ``activations_chunk`` builds one chunk of the activation
recipe (outliers and zero blocks included) from its own child stream of the
seed, so chunks can be built in parallel.

Nothing here is part of the quantization method.
"""

import numpy as np
import torch

BLOCK = 128

# seeds per workload
SEED_TINY = 0
SEED_ACT_QUANT = 1
SEED_DEQUANT = 2
SEED_DEQUANT_RAGGED = 12
SEED_DECODE_BASE = 3      # + M
SEED_PREFILL = (4, 5)     # shape 1, shape 2
SEED_WEIGHT_QUANT = 6
SEED_WEIGHT_QUANT_RAGGED = 16


def rng_for(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def normal_f32(rng, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def add_outliers(rng, x: np.ndarray, frac: float = 1e-3, factor: float = 100.0) -> np.ndarray:
    """Multiply round(frac * numel) distinct, uniformly chosen elements by ``factor``."""
    flat = x.reshape(-1)
    count = int(round(frac * flat.size))
    if count:
        pos = rng.choice(flat.size, size=count, replace=False)
        flat[pos] = flat[pos] * np.float32(factor)
    return x


def zero_one_block_per_row_group(rng, x: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Zero one 1 x block run in every group of 128 rows."""
    rows, k = x.shape
    groups = -(-rows // 128)
    for g in range(groups):
        hi = min(128, rows - 128 * g)
        r = 128 * g + int(rng.integers(0, hi))
        j = int(rng.integers(0, k // block))
        x[r, j * block:(j + 1) * block] = 0.0
    return x


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """fp32 numpy -> bf16 CPU tensor (torch's round-to-nearest-even cast)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


def activations(rng, m: int, k: int, dtype: str = "bf16", outliers: bool = False,
                zero_blocks: bool = False) -> torch.Tensor:
    """Activation matrix [m, k] as a CPU tensor of ``dtype`` ('bf16' or 'f32')."""
    x = normal_f32(rng, (m, k))
    if outliers:
        add_outliers(rng, x)
    if zero_blocks:
        zero_one_block_per_row_group(rng, x)
    if dtype == "bf16":
        return to_bf16(x)
    if dtype == "f32":
        return torch.from_numpy(x)
    raise ValueError(dtype)


def activations_chunk(seed: int, m: int, k: int, index: int, rows_per_chunk: int = 16384):
    """Chunk `index` (rows index * rows_per_chunk onward, as a bf16 CPU tensor) of
    an [m, k] activation matrix too large to build in one piece, with the
    prefill recipe (N(0,1), 0.1% outliers x100, one zero 1 x 128 block per
    128-row group).  Each chunk draws from its own child stream of `seed`
    (SeedSequence spawn key (index,)), so chunks can be built in any order or
    in parallel.  Chunks hold whole 128-row groups."""
    if rows_per_chunk % 128:
        raise ValueError("rows_per_chunk must be a multiple of 128")
    r0 = index * rows_per_chunk
    if not 0 <= r0 < m:
        raise ValueError("chunk index out of range")
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(index,)))
    return activations(rng, min(rows_per_chunk, m - r0), k, outliers=True, zero_blocks=True)


def weight_codes(rng, n: int, k: int) -> np.ndarray:
    """Uniform over the 254 finite E4M3 codes, uint8 [n, k]."""
    c = rng.integers(0, 254, size=(n, k), dtype=np.int16)
    c = np.where(c >= 0x7F, c + 1, c)      # skip 0x7F; 254 -> 255 never drawn
    return c.astype(np.uint8)


def weight_codes_chunks(seed: int, n: int, k: int, rows_per_chunk: int = 32768):
    """The same distribution for matrices too large to build in one piece:
    yields (first row, uint8 [rows, k]) in row order, from one generator
    seeded with `seed`."""
    rng = rng_for(seed)
    for r0 in range(0, n, rows_per_chunk):
        c = rng.integers(0, 254, size=(min(rows_per_chunk, n - r0), k), dtype=np.uint8)
        c += c >= 0x7F                     # skip 0x7F; 254 -> 255 never drawn
        yield r0, c


def log_uniform_scales(rng, shape, lo: float, hi: float) -> np.ndarray:
    return (2.0 ** rng.uniform(lo, hi, size=shape)).astype(np.float32)


def scale_grid(n: int, k: int, block: int = BLOCK):
    return (-(-n // block), -(-k // block))


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

def tiny_gemm():
    """fp32 activations [16, 512] N(0,1); weights [256, 512]; scales 2^U[-12,-4]."""
    rng = rng_for(SEED_TINY)
    x = activations(rng, 16, 512, dtype="f32")
    w = weight_codes(rng, 256, 512)
    ws = log_uniform_scales(rng, scale_grid(256, 512), -12, -4)
    return {"x": x, "w": w, "w_s": ws, "scale_fmt": None, "out": "f32"}


def act_quant_workload(m: int = 8192, k: int = 7168, seed: int = SEED_ACT_QUANT):
    """bf16 [m, k] N(0,1), 0.1% outliers x100, one zero block per 128-row group."""
    rng = rng_for(seed)
    return {"x": activations(rng, m, k, dtype="bf16", outliers=True, zero_blocks=True)}


def dequant_workload(n: int = 18432, k: int = 7168, seed: int = None):
    """E4M3 codes [n, k], scales [ceil(n/128), ceil(k/128)] in 2^U[-14,-2]."""
    if seed is None:
        seed = SEED_DEQUANT if n % BLOCK == 0 else SEED_DEQUANT_RAGGED
    rng = rng_for(seed)
    w = weight_codes(rng, n, k)
    ws = log_uniform_scales(rng, scale_grid(n, k), -14, -2)
    return {"w": w, "w_s": ws}


def decode_gemm(m: int, n: int = 18432, k: int = 7168):
    """bf16 activations [m, k] N(0,1); weights [n, k]; scales 2^U[-14,-2]."""
    rng = rng_for(SEED_DECODE_BASE + m)
    x = activations(rng, m, k, dtype="bf16")
    w = weight_codes(rng, n, k)
    ws = log_uniform_scales(rng, scale_grid(n, k), -14, -2)
    return {"x": x, "w": w, "w_s": ws, "scale_fmt": None, "out": "bf16"}


def prefill_gemm(shape: int = 1, m: int = 8192):
    """Shape 1: [m, 7168] x [18432, 7168]; shape 2: [m, 18432] x [7168, 18432]."""
    n, k = (18432, 7168) if shape == 1 else (7168, 18432)
    rng = rng_for(SEED_PREFILL[shape - 1])
    x = activations(rng, m, k, dtype="bf16", outliers=True)
    w = weight_codes(rng, n, k)
    ws = log_uniform_scales(rng, scale_grid(n, k), -14, -2)
    return {"x": x, "w": w, "w_s": ws, "scale_fmt": "ue8m0", "out": "bf16"}


def weight_quant_workload(n: int = 18432, k: int = 7168, seed: int = None, dtype: str = "bf16"):
    """Weights [n, k] to quantize per 128 x 128 tile (``dtype`` 'bf16' or 'f32')."""
    if seed is None:
        seed = SEED_WEIGHT_QUANT if n % BLOCK == 0 and k % BLOCK == 0 else SEED_WEIGHT_QUANT_RAGGED
    rng = rng_for(seed)
    gm, gn = scale_grid(n, k)
    w = normal_f32(rng, (n, k))
    mag = log_uniform_scales(rng, (gm, gn), -10, 0)
    w *= np.repeat(np.repeat(mag, BLOCK, 0), BLOCK, 1)[:n, :k]
    add_outliers(rng, w, frac=1e-4)
    for i in range(0, gm, 8):
        j = int(rng.integers(0, gn))
        w[i * BLOCK:(i + 1) * BLOCK, j * BLOCK:(j + 1) * BLOCK] = 0.0
    if dtype == "bf16":
        return {"w": to_bf16(w)}
    if dtype == "f32":
        return {"w": torch.from_numpy(w)}
    raise ValueError(dtype)


def custom_gemm(seed: int, m: int, n: int, k: int, dtype: str = "bf16", outliers: bool = False,
                lo: float = -14, hi: float = -2):
    """Arbitrary-shape GEMM inputs, same recipe (for ragged and edge cases)."""
    rng = rng_for(seed)
    x = activations(rng, m, k, dtype=dtype, outliers=outliers)
    w = weight_codes(rng, n, k)
    ws = log_uniform_scales(rng, scale_grid(n, k), lo, hi)
    return {"x": x, "w": w, "w_s": ws}


__all__ = [name for name in dir() if not name.startswith("_") and name not in ("np", "torch")]
