"""Loading ``libfp8bsq.so`` and declaring its C ABI for ctypes.

The library is built in-tree (``python -m fp8_block_scaled_quant_amd.build``
or ``__graft_entry__.build()``).  Loading it initializes nothing on the GPU.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8bsq.so")

# enums of include/fp8bsq.h
OK, EINVAL, ESHAPE, EUNSUPPORTED, EALIGN, ELAUNCH, ERANGE, ESCRATCH = range(8)
SPLIT_SCRATCH_BYTES = 67109376   # FP8BSQ_SPLIT_SCRATCH_BYTES
F32, BF16 = 0, 1
SCALE_NONE, SCALE_UE8M0 = 0, 1

# every symbol include/fp8bsq.h declares
EXPORTS = ("fp8_act_quant", "fp8_weight_dequant", "fp8_weight_quant", "fp8_block_gemm",
           "fp8_block_gemm_ue8m0", "fp8_block_gemm_reference", "fp8_block_gemm_split",
           "fp8_block_gemm_split_workspace", "fp8_block_gemm_split_noalloc", "fp8_act_quant_gemm",
           "fp8bsq_strerror", "fp8bsq_version")

_LIB = None


class Fp8Error(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"fp8bsq status {status}: {text}")
        self.status = status


def library_path() -> str:
    return LIB_PATH


def load_library(path: str = None) -> ctypes.CDLL:
    """Load the shared library and declare argument types; raises if absent."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(
            f"{p} is missing: build the HIP library first (python -m fp8_block_scaled_quant_amd.build)")
    lib = ctypes.CDLL(p)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.fp8_act_quant.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, vp]
    lib.fp8_act_quant.restype = i32
    lib.fp8_weight_dequant.argtypes = [vp, vp, i64, i64, i32, vp, i32, vp]
    lib.fp8_weight_dequant.restype = i32
    lib.fp8_weight_quant.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, vp]
    lib.fp8_weight_quant.restype = i32
    lib.fp8_block_gemm.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, vp]
    lib.fp8_block_gemm.restype = i32
    lib.fp8_block_gemm_ue8m0.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, vp]
    lib.fp8_block_gemm_ue8m0.restype = i32
    lib.fp8_block_gemm_reference.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, vp]
    lib.fp8_block_gemm_reference.restype = i32
    lib.fp8_block_gemm_split.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, i32, vp,
                                         ctypes.c_size_t, vp]
    lib.fp8_block_gemm_split.restype = i32
    lib.fp8_block_gemm_split_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, i32, vp]
    lib.fp8_block_gemm_split_noalloc.restype = i32
    lib.fp8_block_gemm_split_workspace.argtypes = [i64, i64, i64]
    lib.fp8_block_gemm_split_workspace.restype = ctypes.c_size_t
    lib.fp8_act_quant_gemm.argtypes = [vp, i32, i32, vp, vp, vp, vp, i32, i64, i64, i64, vp, vp, vp]
    lib.fp8_act_quant_gemm.restype = i32
    lib.fp8bsq_strerror.argtypes = [i32]
    lib.fp8bsq_strerror.restype = ctypes.c_char_p
    lib.fp8bsq_version.argtypes = []
    lib.fp8bsq_version.restype = ctypes.c_char_p
    if path is None:
        _LIB = lib
    return lib


def lib() -> ctypes.CDLL:
    return load_library()


def check(status: int):
    if status != OK:
        raise Fp8Error(status, lib().fp8bsq_strerror(status).decode())
