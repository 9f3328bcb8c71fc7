"""Helpers for the GPU parity tests: direct C-ABI calls with guard bands.

Every output buffer is allocated with 4 KiB of canary bytes on each side; after
the call the canaries must be untouched (an out-of-bounds write on a ragged edge
would show up there).
"""

import ctypes

import numpy as np
import torch

from fp8_block_scaled_quant_amd import _lib

GUARD = 4096
CANARY = 0xA5


def device() -> torch.device:
    if not torch.cuda.is_available():
        raise RuntimeError("GPU parity tests need a ROCm GPU (gfx950)")
    return torch.device("cuda:0")


class Guarded:
    """A uint8 device buffer of `nbytes` surrounded by canary bytes."""

    def __init__(self, nbytes: int, offset: int = 0):
        self.nbytes = nbytes
        self.offset = offset
        self.buf = torch.full((nbytes + 2 * GUARD + offset,), CANARY, dtype=torch.uint8, device=device())
        self.ptr = self.buf.data_ptr() + GUARD + offset

    def payload(self) -> torch.Tensor:
        return self.buf[GUARD + self.offset:GUARD + self.offset + self.nbytes]

    def check_guards(self):
        head = self.buf[:GUARD + self.offset]
        tail = self.buf[GUARD + self.offset + self.nbytes:]
        assert bool((head == CANARY).all()), "write before the output buffer"
        assert bool((tail == CANARY).all()), "write past the end of the output buffer"


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def act_quant(x: torch.Tensor, scale_fmt=None):
    """x: CUDA bf16/fp32 [rows, k].  Returns (codes uint8 numpy, scales fp32 numpy)."""
    rows, k = x.shape
    y = Guarded(rows * k)
    s = Guarded(rows * (k // 128) * 4)
    dt = _lib.BF16 if x.dtype == torch.bfloat16 else _lib.F32
    fmt = _lib.SCALE_UE8M0 if scale_fmt == "ue8m0" else _lib.SCALE_NONE
    st = _lib.lib().fp8_act_quant(ctypes.c_void_p(x.data_ptr()), dt, rows, k, 128, fmt,
                                  ctypes.c_void_p(y.ptr), ctypes.c_void_p(s.ptr), stream())
    assert st == _lib.OK, st
    torch.cuda.synchronize()
    y.check_guards()
    s.check_guards()
    codes = y.payload().cpu().numpy().reshape(rows, k)
    scales = s.payload().cpu().numpy().view(np.float32).reshape(rows, k // 128)
    return codes, scales


def weight_quant(w: torch.Tensor, scale_fmt=None, offset: int = 0):
    """w: CUDA bf16/fp32 [m, n] (moved to a buffer offset by `offset` elements).

    Returns (codes uint8 numpy [m, n], scales fp32 numpy grid).
    """
    m, n = w.shape
    esz = w.element_size()
    wd = Guarded(m * n * esz, offset=offset * esz)
    wd.payload().copy_(w.contiguous().view(torch.uint8).reshape(-1))
    gm, gn = -(-m // 128), -(-n // 128)
    y = Guarded(m * n, offset=offset)
    s = Guarded(gm * gn * 4)
    dt = _lib.BF16 if w.dtype == torch.bfloat16 else _lib.F32
    fmt = _lib.SCALE_UE8M0 if scale_fmt == "ue8m0" else _lib.SCALE_NONE
    st = _lib.lib().fp8_weight_quant(ctypes.c_void_p(wd.ptr), dt, m, n, 128, fmt,
                                     ctypes.c_void_p(y.ptr), ctypes.c_void_p(s.ptr), stream())
    assert st == _lib.OK, st
    torch.cuda.synchronize()
    y.check_guards()
    s.check_guards()
    wd.check_guards()
    return (y.payload().cpu().numpy().reshape(m, n),
            s.payload().cpu().numpy().view(np.float32).reshape(gm, gn))


def weight_dequant(w: np.ndarray, s: np.ndarray, out: str = "bf16", offset: int = 0):
    """w uint8 [m, n], s fp32 grid.  Returns bf16 bits (uint16) or fp32 numpy."""
    m, n = w.shape
    dev = device()
    wd = Guarded(m * n, offset=offset)
    wd.payload().copy_(torch.from_numpy(w.reshape(-1)).to(dev))
    sd = torch.from_numpy(s).to(dev)
    esz = 2 if out == "bf16" else 4
    y = Guarded(m * n * esz, offset=offset * esz)
    st = _lib.lib().fp8_weight_dequant(ctypes.c_void_p(wd.ptr), ctypes.c_void_p(sd.data_ptr()), m, n,
                                       128, ctypes.c_void_p(y.ptr), _lib.BF16 if out == "bf16" else _lib.F32,
                                       stream())
    assert st == _lib.OK, st
    torch.cuda.synchronize()
    y.check_guards()
    raw = y.payload().cpu().numpy()
    return raw.view(np.uint16).reshape(m, n) if out == "bf16" else raw.view(np.float32).reshape(m, n)


def block_gemm(a: np.ndarray, a_s: np.ndarray, b: np.ndarray, b_s: np.ndarray, out: str = "bf16",
               a_dev: torch.Tensor = None, a_s_dev: torch.Tensor = None, ue8m0: bool = False,
               entry: str = None):
    """Returns C as float64 numpy (bf16 widened exactly).

    ``entry`` names the C entry point (default fp8_block_gemm, or
    fp8_block_gemm_ue8m0 when ``ue8m0``)."""
    dev = device()
    m, k = a.shape if a is not None else a_dev.shape
    n = b.shape[0]
    ad = a_dev if a_dev is not None else torch.from_numpy(a).to(dev)
    asd = a_s_dev if a_s_dev is not None else torch.from_numpy(a_s).to(dev)
    bd = torch.from_numpy(b).to(dev)
    bsd = torch.from_numpy(b_s).to(dev)
    esz = 2 if out == "bf16" else 4
    c = Guarded(m * n * esz)
    if entry is None:
        entry = "fp8_block_gemm_ue8m0" if ue8m0 else "fp8_block_gemm"
    fn = getattr(_lib.lib(), entry)
    st = fn(ctypes.c_void_p(ad.data_ptr()), ctypes.c_void_p(asd.data_ptr()),
                                   ctypes.c_void_p(bd.data_ptr()), ctypes.c_void_p(bsd.data_ptr()),
                                   ctypes.c_void_p(c.ptr), _lib.BF16 if out == "bf16" else _lib.F32,
                                   m, n, k, stream())
    assert st == _lib.OK, st
    torch.cuda.synchronize()
    c.check_guards()
    raw = c.payload().cpu().numpy()
    if out == "bf16":
        bits = raw.view(np.uint16).reshape(m, n).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    return raw.view(np.float32).reshape(m, n).astype(np.float64)


def act_quant_gemm(x: torch.Tensor, b: np.ndarray, b_s: np.ndarray, scale_fmt=None, out: str = "bf16",
                   bias: torch.Tensor = None):
    """Fused entry point.  x: CUDA bf16/fp32 [m, k].

    Returns (C float64 numpy, codes uint8 numpy, scales fp32 numpy).
    """
    dev = device()
    m, k = x.shape
    n = b.shape[0]
    bd = torch.from_numpy(b).to(dev)
    bsd = torch.from_numpy(b_s).to(dev)
    esz = 2 if out == "bf16" else 4
    c = Guarded(m * n * esz)
    y = Guarded(m * k)
    s = Guarded(m * (k // 128) * 4)
    dt = _lib.BF16 if x.dtype == torch.bfloat16 else _lib.F32
    fmt = _lib.SCALE_UE8M0 if scale_fmt == "ue8m0" else _lib.SCALE_NONE
    st = _lib.lib().fp8_act_quant_gemm(ctypes.c_void_p(x.data_ptr()), dt, fmt,
                                       ctypes.c_void_p(bd.data_ptr()), ctypes.c_void_p(bsd.data_ptr()),
                                       ctypes.c_void_p(None if bias is None else bias.data_ptr()),
                                       ctypes.c_void_p(c.ptr), _lib.BF16 if out == "bf16" else _lib.F32,
                                       m, n, k, ctypes.c_void_p(y.ptr), ctypes.c_void_p(s.ptr), stream())
    assert st == _lib.OK, st
    torch.cuda.synchronize()
    for g in (c, y, s):
        g.check_guards()
    raw = c.payload().cpu().numpy()
    if out == "bf16":
        got = ((raw.view(np.uint16).reshape(m, n).astype(np.uint32) << 16).view(np.float32)).astype(np.float64)
    else:
        got = raw.view(np.float32).reshape(m, n).astype(np.float64)
    return (got, y.payload().cpu().numpy().reshape(m, k),
            s.payload().cpu().numpy().view(np.float32).reshape(m, k // 128))


def announce(msg: str):
    print(f"[gpu-test] {msg}", flush=True)


def block_gemm_split(a_dev: torch.Tensor, a_s_dev: torch.Tensor, b: np.ndarray, b_s: np.ndarray,
                     out: str = "bf16", ue8m0: bool = False, ws: "Guarded" = None, ws_bytes: int = None):
    """fp8_block_gemm_split with a canary-guarded output and workspace.

    ws_bytes defaults to what fp8_block_gemm_split_workspace asks for; pass
    ws to reuse a workspace (its contents are left as the last call left
    them).  Returns (C as float64 numpy, the workspace).
    """
    dev = device()
    m, k = a_dev.shape
    n = b.shape[0]
    bd = torch.from_numpy(b).to(dev)
    bsd = torch.from_numpy(b_s).to(dev)
    lib = _lib.lib()
    need = lib.fp8_block_gemm_split_workspace(m, n, k)
    if ws is None:
        ws = Guarded(max(need if ws_bytes is None else ws_bytes, 256))
    nbytes = ws.nbytes if ws_bytes is None else ws_bytes
    esz = 2 if out == "bf16" else 4
    c = Guarded(m * n * esz)
    st = lib.fp8_block_gemm_split(ctypes.c_void_p(a_dev.data_ptr()), ctypes.c_void_p(a_s_dev.data_ptr()),
                                  ctypes.c_void_p(bd.data_ptr()), ctypes.c_void_p(bsd.data_ptr()),
                                  ctypes.c_void_p(c.ptr), _lib.BF16 if out == "bf16" else _lib.F32, m, n, k,
                                  _lib.SCALE_UE8M0 if ue8m0 else _lib.SCALE_NONE, ctypes.c_void_p(ws.ptr),
                                  nbytes, stream())
    assert st == _lib.OK, st
    torch.cuda.synchronize()
    c.check_guards()
    ws.check_guards()
    raw = c.payload().cpu().numpy()
    if out == "bf16":
        bits = raw.view(np.uint16).reshape(m, n).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64), ws
    return raw.view(np.float32).reshape(m, n).astype(np.float64), ws
