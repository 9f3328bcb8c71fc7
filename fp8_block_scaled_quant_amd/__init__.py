"""Block-scaled FP8 (E4M3) quantization and GEMM on AMD Instinct MI355X.

A thin ctypes binding over the C ABI of ``libfp8bsq.so`` (declared in
``include/fp8bsq.h``).  PyTorch supplies device memory and the current stream;
every step of the computation runs in the library's HIP kernels.  There is no
fallback: if the library is not built, or a tensor is not on a GPU, the calls
raise.

Functions follow the call shapes the pages give:

* ``act_quant(x, block_size=128, scale_fmt=None) -> (y, s)``
* ``weight_dequant(x, s, block_size=128, out_dtype=torch.float32) -> y``
* ``fp8_gemm(a, a_s, b, b_s, out_dtype=torch.bfloat16, scale_fmt=None) -> c``
  (``scale_fmt="ue8m0"`` declares a_s powers of two: they are then applied
  inside the MX-scaled MFMA, with a bit-identical result)

and, producing the GEMM's weight operand,

* ``weight_quant(w, block_size=128, scale_fmt=None) -> (y, s)``

and a linear layer's forward product in one call (act_quant, then fp8_gemm;
a single kernel for bf16 decode batches of up to 16 rows),

* ``act_quant_gemm(x, b, b_s, scale_fmt=None, out_dtype=torch.bfloat16, bias=None) -> (c, y, s)``

``Linear`` (in ``fp8_block_scaled_quant_amd.linear``) wraps the last one as a
``torch.nn.Module`` holding an E4M3 weight and its 128x128 block scales.
"""

import ctypes

import torch

from . import _lib

__all__ = ["act_quant", "weight_dequant", "weight_quant", "fp8_gemm", "act_quant_gemm", "Linear",
           "Fp8Error", "library_path", "load_library"]

Fp8Error = _lib.Fp8Error
library_path = _lib.library_path
load_library = _lib.load_library

_DTYPE = {torch.float32: _lib.F32, torch.bfloat16: _lib.BF16}
_SCALE_FMT = {None: _lib.SCALE_NONE, "ue8m0": _lib.SCALE_UE8M0}


def _stream_handle(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _require_gpu(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("fp8_block_scaled_quant_amd runs on the GPU only: tensor is on " + str(t.device))
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    dev = ts[0].device
    if any(t.device != dev for t in ts):
        raise ValueError("all tensors must be on the same device")


def _codes(t: torch.Tensor) -> torch.Tensor:
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    if t.dtype == torch.uint8:
        return t
    raise TypeError("E4M3 operands must be torch.float8_e4m3fn (or uint8 codes)")


def act_quant(x: torch.Tensor, block_size: int = 128, scale_fmt=None):
    """Dynamic activation quantization: one FP32 scale per 1 x block_size block.

    ``x`` is a contiguous bf16 or fp32 CUDA tensor whose last dimension is a
    multiple of ``block_size``.  Returns ``y`` (float8_e4m3fn, x's shape) and
    ``s`` (float32, ``x.shape[:-1] + (K // block_size,)``).
    """
    _require_gpu(x)
    if x.dtype not in _DTYPE:
        raise TypeError("act_quant takes bf16 or fp32 input")
    if scale_fmt not in _SCALE_FMT:
        raise ValueError(f"unknown scale_fmt {scale_fmt!r}")
    k = x.shape[-1]
    if k % block_size != 0:
        raise ValueError("last dimension must be a multiple of block_size")
    rows = x.numel() // k if k else 0
    y = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    s = torch.empty(x.shape[:-1] + (k // block_size,), dtype=torch.float32, device=x.device)
    if rows:
        _lib.check(_lib.lib().fp8_act_quant(
            ctypes.c_void_p(x.data_ptr()), _DTYPE[x.dtype], rows, k, block_size,
            _SCALE_FMT[scale_fmt], ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(s.data_ptr()),
            _stream_handle(x)))
    return y.view(torch.float8_e4m3fn), s


def weight_dequant(x: torch.Tensor, s: torch.Tensor, block_size: int = 128,
                   out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Dequantize a 2-D E4M3 weight with its [ceil(M/bs), ceil(N/bs)] FP32 block scales."""
    x = _codes(x)
    _require_gpu(x, s)
    if x.dim() != 2:
        raise ValueError("weight must be 2-D")
    if s.dtype != torch.float32:
        raise TypeError("scales must be float32")
    if out_dtype not in _DTYPE:
        raise TypeError("out_dtype must be float32 or bfloat16")
    m, n = x.shape
    grid = (-(-m // block_size), -(-n // block_size))
    if tuple(s.shape) != grid:
        raise ValueError(f"scale grid must be {grid}, got {tuple(s.shape)}")
    y = torch.empty((m, n), dtype=out_dtype, device=x.device)
    if m and n:
        _lib.check(_lib.lib().fp8_weight_dequant(
            ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(s.data_ptr()), m, n, block_size,
            ctypes.c_void_p(y.data_ptr()), _DTYPE[out_dtype], _stream_handle(x)))
    return y


def weight_quant(w: torch.Tensor, block_size: int = 128, scale_fmt=None):
    """Quantize a 2-D weight per block_size x block_size tile.

    ``w`` is a contiguous bf16 or fp32 CUDA tensor [M, N] (any M, N >= 0).
    Returns ``y`` (float8_e4m3fn [M, N]) and ``s`` (float32
    [ceil(M/bs), ceil(N/bs)]), the operands ``weight_dequant`` and ``fp8_gemm``
    take.
    """
    _require_gpu(w)
    if w.dtype not in _DTYPE:
        raise TypeError("weight_quant takes bf16 or fp32 input")
    if w.dim() != 2:
        raise ValueError("weight must be 2-D")
    if scale_fmt not in _SCALE_FMT:
        raise ValueError(f"unknown scale_fmt {scale_fmt!r}")
    m, n = w.shape
    y = torch.empty((m, n), dtype=torch.uint8, device=w.device)
    s = torch.empty((-(-m // block_size), -(-n // block_size)), dtype=torch.float32, device=w.device)
    if m and n:
        _lib.check(_lib.lib().fp8_weight_quant(
            ctypes.c_void_p(w.data_ptr()), _DTYPE[w.dtype], m, n, block_size, _SCALE_FMT[scale_fmt],
            ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(s.data_ptr()), _stream_handle(w)))
    return y.view(torch.float8_e4m3fn), s


def fp8_gemm(a: torch.Tensor, a_s: torch.Tensor, b: torch.Tensor, b_s: torch.Tensor,
             out_dtype: torch.dtype = torch.bfloat16, scale_fmt=None, split: bool = True) -> torch.Tensor:
    """Block-scaled FP8 GEMM ``C = A . B^T`` (B is the [out, in] weight).

    ``a`` [..., K] E4M3 with ``a_s`` [..., K/128]; ``b`` [N, K] E4M3 with
    ``b_s`` [ceil(N/128), K/128].  Returns ``[..., N]`` in ``out_dtype``.
    ``scale_fmt="ue8m0"`` states that every a_s is a power of two (act_quant's
    ue8m0 scales) and selects the entry point that applies them in the MFMA.
    ``split`` (default) lets a last round of output tiles that would leave
    compute units idle run split over K (fp8_block_gemm_split, with a workspace
    from torch's allocator); results then differ from ``split=False`` only in
    FP32 summation order.
    """
    if scale_fmt not in _SCALE_FMT:
        raise ValueError(f"unknown scale_fmt {scale_fmt!r}")
    a, b = _codes(a), _codes(b)
    _require_gpu(a, a_s, b, b_s)
    if a_s.dtype != torch.float32 or b_s.dtype != torch.float32:
        raise TypeError("scales must be float32")
    if out_dtype not in _DTYPE:
        raise TypeError("out_dtype must be float32 or bfloat16")
    k = a.shape[-1]
    if b.dim() != 2 or b.shape[1] != k:
        raise ValueError("b must be [N, K] with A's K")
    if k <= 0 or k % 128 != 0:
        raise ValueError("K must be a positive multiple of 128")
    m = a.numel() // k
    n = b.shape[0]
    if tuple(a_s.shape) != tuple(a.shape[:-1]) + (k // 128,):
        raise ValueError("a_s must be a.shape[:-1] + (K/128,)")
    if tuple(b_s.shape) != (-(-n // 128), k // 128):
        raise ValueError("b_s must be [ceil(N/128), K/128]")
    c = torch.empty(tuple(a.shape[:-1]) + (n,), dtype=out_dtype, device=a.device)
    if m and n:
        lib = _lib.lib()
        args = (ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(a_s.data_ptr()),
                ctypes.c_void_p(b.data_ptr()), ctypes.c_void_p(b_s.data_ptr()),
                ctypes.c_void_p(c.data_ptr()), _DTYPE[out_dtype], m, n, k)
        ws_bytes = lib.fp8_block_gemm_split_workspace(m, n, k) if split else 0
        if ws_bytes:
            # scratch for the split-K tail; torch's allocator keeps it from being
            # reused until the work queued on this stream has passed it
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=a.device)
            _lib.check(lib.fp8_block_gemm_split(*args, _SCALE_FMT[scale_fmt], ctypes.c_void_p(ws.data_ptr()),
                                                ws_bytes, _stream_handle(a)))
        else:
            fn = lib.fp8_block_gemm_ue8m0 if scale_fmt == "ue8m0" else lib.fp8_block_gemm
            _lib.check(fn(*args, _stream_handle(a)))
    return c


def act_quant_gemm(x: torch.Tensor, b: torch.Tensor, b_s: torch.Tensor, scale_fmt=None,
                   out_dtype: torch.dtype = torch.bfloat16, bias: torch.Tensor = None):
    """``act_quant(x)`` then ``fp8_gemm`` with the weight ``b`` [N, K] / ``b_s``.

    ``bias`` ([N], ``out_dtype``) is added to the FP32 accumulator before the
    output rounding.  Returns ``(c [..., N], y, s)`` where ``(y, s)`` are
    act_quant's outputs, bit-identical to calling ``act_quant`` separately.
    """
    b = _codes(b)
    _require_gpu(x, b, b_s, *(() if bias is None else (bias,)))
    if x.dtype not in _DTYPE:
        raise TypeError("act_quant_gemm takes bf16 or fp32 activations")
    if scale_fmt not in _SCALE_FMT:
        raise ValueError(f"unknown scale_fmt {scale_fmt!r}")
    if out_dtype not in _DTYPE:
        raise TypeError("out_dtype must be float32 or bfloat16")
    if b_s.dtype != torch.float32:
        raise TypeError("scales must be float32")
    k = x.shape[-1]
    if k <= 0 or k % 128 != 0:
        raise ValueError("K must be a positive multiple of 128")
    if b.dim() != 2 or b.shape[1] != k:
        raise ValueError("b must be [N, K] with x's K")
    n = b.shape[0]
    if tuple(b_s.shape) != (-(-n // 128), k // 128):
        raise ValueError("b_s must be [ceil(N/128), K/128]")
    if bias is not None and (bias.dtype != out_dtype or tuple(bias.shape) != (n,)):
        raise ValueError(f"bias must be [{n}] of the output dtype {out_dtype}")
    m = x.numel() // k
    y = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    s = torch.empty(x.shape[:-1] + (k // 128,), dtype=torch.float32, device=x.device)
    c = torch.empty(tuple(x.shape[:-1]) + (n,), dtype=out_dtype, device=x.device)
    if m:   # with n = 0 the library still writes y and s
        _lib.check(_lib.lib().fp8_act_quant_gemm(
            ctypes.c_void_p(x.data_ptr()), _DTYPE[x.dtype], _SCALE_FMT[scale_fmt],
            ctypes.c_void_p(b.data_ptr()), ctypes.c_void_p(b_s.data_ptr()),
            ctypes.c_void_p(None if bias is None else bias.data_ptr()),
            ctypes.c_void_p(c.data_ptr()), _DTYPE[out_dtype], m, n, k,
            ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(s.data_ptr()), _stream_handle(x)))
    return c, y.view(torch.float8_e4m3fn), s


from .linear import Linear  # noqa: E402  (uses the functions above)
