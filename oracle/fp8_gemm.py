"""Block-scaled FP8 GEMM and its error bound (oracle; test infrastructure only).

What the pages fix:

* ``fp8_gemm(a, a_s, b, b_s)`` takes activation codes with their per-block
  scales and weight codes with their 128x128 block scales, in the same per-block
  layouts act_quant and weight_dequant use, and folds the scaling into the
  matrix product instead of materializing dequantized weights (page "How
  weight_dequant Handles Per-Block Scaling in DeepSeek-V3 FP8 GEMM", section
  "Relationship to FP8 GEMM Operations").
* weights are used as in ``F.linear(x, W)``, i.e. W is [out, in] and the
  product is x @ W^T (same page, "Practical Usage Example").
* partial sums are periodically promoted to FP32 (page "DeepSeek-V3: How
  Selective FP8 Stays Stable", "Learning outcomes" and FAQ), and outputs are
  BF16 or FP32 (same page, "Lower precision is a constrained budget").

Readings:
  R13 A [M, K] and B [N, K] row-major, C = A . B^T; a_s [M, K/128] (act_quant's
      layout), b_s [ceil(N/128), K/128] (weight_dequant's grid).
  R14 the promotion interval is the 128-wide K block: for each K block kb,
      P = sum over the block of DEC(A) * DEC(B), then C += P * (a_s * b_s).
  R15 accumulation order on the GPU is free; results are held to the bound in
      ``gemm_tolerance`` (1e-3 * sum_k |a_k b_k|, plus one BF16 ulp for BF16).
  R16 BF16 output is the FP32 accumulator rounded to nearest even.

The oracle works in float64.  Each block partial P is exact in any order: an
E4M3 x E4M3 product is a multiple of 2^-18 below 2^18, so 128 of them sum to
fewer than 2^43 units of 2^-18, within float64's 53 bits.  The scale product of
two FP32 values is exact in float64 too; the only roundings are one multiply
and one add per K block.
"""

import numpy as np

from . import e4m3


def _rows(a, rows):
    return a if rows is None else a[np.asarray(rows)]


def _check(a, a_s, b, b_s, block_size):
    if a.dtype != np.uint8 or b.dtype != np.uint8:
        raise TypeError("A and B must be uint8 E4M3 codes")
    if a_s.dtype != np.float32 or b_s.dtype != np.float32:
        raise TypeError("scales must be float32")
    m, k = a.shape
    n, k2 = b.shape
    if k != k2 or k % block_size:
        raise ValueError("A and B must share K, a multiple of the block size")
    kb = k // block_size
    if a_s.shape != (m, kb):
        raise ValueError(f"a_s must be {(m, kb)}")
    if b_s.shape != (-(-n // block_size), kb):
        raise ValueError(f"b_s must be {(-(-n // block_size), kb)}")
    return m, n, k, kb


def fp8_gemm(a, a_s, b, b_s, block_size: int = 128, rows=None) -> np.ndarray:
    """C[m, n] = sum_kb P_kb[m, n] * a_s[m, kb] * b_s[n // bs, kb], float64.

    ``rows`` (optional index array) restricts the result to those rows of A,
    so full-size problems can be checked on sampled rows.
    """
    m, n, k, nkb = _check(a, a_s, b, b_s, block_size)
    a = _rows(a, rows)
    a_s = _rows(a_s, rows)
    c = np.zeros((a.shape[0], n), dtype=np.float64)
    col_block = np.arange(n) // block_size
    for kb in range(nkb):
        ks = slice(kb * block_size, (kb + 1) * block_size)
        pa = e4m3.decode(a[:, ks])                       # [m, bs] float64
        pb = e4m3.decode(b[:, ks])                       # [n, bs] float64
        partial = pa @ pb.T                              # exact block partial
        scale = a_s[:, kb].astype(np.float64)[:, None] * b_s[col_block, kb].astype(np.float64)[None, :]
        c += partial * scale
    return c


def dequantized_operands(a, a_s, b, b_s, block_size: int = 128, rows=None):
    """A_hat = DEC(A) * a_s and B_hat = DEC(B) * b_s elementwise, float64 (exact)."""
    m, n, k, nkb = _check(a, a_s, b, b_s, block_size)
    a = _rows(a, rows)
    a_s = _rows(a_s, rows)
    a_hat = e4m3.decode(a) * np.repeat(a_s.astype(np.float64), block_size, axis=1)
    b_scale = np.repeat(np.repeat(b_s.astype(np.float64), block_size, axis=0)[:n], block_size, axis=1)
    b_hat = e4m3.decode(b) * b_scale
    return a_hat, b_hat


def gemm_tolerance(a, a_s, b, b_s, block_size: int = 128, rows=None, rel: float = 1e-3) -> np.ndarray:
    """Per-element bound rel * sum_k |A_hat[m, k] * B_hat[n, k]|, float64."""
    a_hat, b_hat = dequantized_operands(a, a_s, b, b_s, block_size, rows)
    return rel * (np.abs(a_hat) @ np.abs(b_hat).T)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """One bf16 ulp at the magnitude of v (float64): the spacing of bf16 values
    in the binade holding |v|.

    bf16 keeps 8 significant bits, so in the binade [2^e, 2^(e+1)) the spacing
    is 2^(e - 7); below the smallest normal 2^-126 (and at zero) it is the
    subnormal spacing 2^-133.  The exponent e = floor(log2 |v|) is taken from
    frexp (|v| = f * 2^E with f in [0.5, 1), so e = E - 1), which is exact for
    every float64; a rounded log2 is not, just below a power of two.
    """
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, big_e = np.frexp(a)
    e = np.where(a > 0, big_e.astype(np.int64) - 1, -126)
    e = np.maximum(e, -126)
    return np.ldexp(1.0, e - 7)


def gemm_check(gpu: np.ndarray, c: np.ndarray, tol: np.ndarray, out: str = "f32") -> np.ndarray:
    """Boolean mask of elements meeting the bound; NaN/Inf always fail."""
    gpu = np.asarray(gpu, dtype=np.float64)
    err = np.abs(gpu - c)
    bound = tol + (bf16_ulp(c) if out == "bf16" else 0.0)
    return np.isfinite(gpu) & (err <= bound)
