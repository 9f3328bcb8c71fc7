"""C-ABI checks that need no GPU: the library loads, exports exactly the
symbols include/fp8bsq.h declares, and rejects bad arguments with the
documented status codes before touching HIP (no kernel is launched here; the
pointers passed are never dereferenced because validation fails first)."""

import os
import re
import subprocess

import pytest

from fp8_block_scaled_quant_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bsq.h")


def declared_symbols():
    text = open(HEADER).read()
    return set(re.findall(r"^FP8BSQ_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M))


@pytest.fixture(scope="module")
def lib():
    return _lib.load_library()


def test_header_declares_entry_points():
    assert declared_symbols() == set(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True)
    exported = {line.split()[-1] for line in out.stdout.splitlines() if " T " in line}
    public = {s for s in exported if not s.startswith("_")}
    assert public == declared_symbols()
    for name in declared_symbols():
        assert getattr(lib, name) is not None


def test_header_enums_match_binding():
    text = open(HEADER).read()
    for name, val in [("FP8BSQ_OK", _lib.OK), ("FP8BSQ_EINVAL", _lib.EINVAL), ("FP8BSQ_ESHAPE", _lib.ESHAPE),
                      ("FP8BSQ_EUNSUPPORTED", _lib.EUNSUPPORTED), ("FP8BSQ_EALIGN", _lib.EALIGN),
                      ("FP8BSQ_ELAUNCH", _lib.ELAUNCH), ("FP8BSQ_ERANGE", _lib.ERANGE),
                      ("FP8BSQ_F32", _lib.F32), ("FP8BSQ_BF16", _lib.BF16),
                      ("FP8BSQ_SCALE_NONE", _lib.SCALE_NONE), ("FP8BSQ_SCALE_UE8M0", _lib.SCALE_UE8M0)]:
        assert re.search(rf"\b{name}\s*=\s*{val}\b", text), name


def test_strerror_and_version(lib):
    for st in range(7):
        assert lib.fp8bsq_strerror(st)
    assert lib.fp8bsq_strerror(99) == b"unknown status"
    assert re.match(rb"^\d+\.\d+\.\d+$", lib.fp8bsq_version())


P = 4096  # a fake, 4096-aligned non-null address: never dereferenced (validation fails first)


def test_act_quant_validation(lib):
    f = lib.fp8_act_quant
    assert f(None, 1, 8, 256, 128, 0, P, P, None) == _lib.EINVAL
    assert f(P, 1, 8, 256, 128, 0, None, P, None) == _lib.EINVAL
    assert f(P, 1, 0, 256, 128, 0, P, P, None) == _lib.EINVAL
    assert f(P, 1, 8, -128, 128, 0, P, P, None) == _lib.EINVAL
    assert f(P, 7, 8, 256, 128, 0, P, P, None) == _lib.EINVAL
    assert f(P, 1, 8, 256, 128, 5, P, P, None) == _lib.EINVAL
    assert f(P, 1, 8, 256, 64, 0, P, P, None) == _lib.EUNSUPPORTED
    assert f(P, 1, 8, 200, 128, 0, P, P, None) == _lib.ESHAPE
    assert f(P + 4, 1, 8, 256, 128, 0, P, P, None) == _lib.EALIGN
    assert f(P, 1, 8, 256, 128, 0, P + 4, P, None) == _lib.EALIGN
    assert f(P, 1, 1 << 31, 256, 128, 0, P, P, None) == _lib.ERANGE


def test_weight_dequant_validation(lib):
    f = lib.fp8_weight_dequant
    assert f(None, P, 8, 8, 128, P, 1, None) == _lib.EINVAL
    assert f(P, P, 0, 8, 128, P, 1, None) == _lib.EINVAL
    assert f(P, P, 8, 8, 128, P, 3, None) == _lib.EINVAL
    assert f(P, P, 8, 8, 256, P, 1, None) == _lib.EUNSUPPORTED
    assert f(P, P + 2, 8, 8, 128, P, 1, None) == _lib.EALIGN
    assert f(P, P, 8, 8, 128, P + 2, 0, None) == _lib.EALIGN
    assert f(P, P, 1 << 31, 8, 128, P, 1, None) == _lib.ERANGE


@pytest.mark.parametrize("name", ["fp8_block_gemm", "fp8_block_gemm_ue8m0"])
def test_block_gemm_validation(lib, name):
    f = getattr(lib, name)
    assert f(None, P, P, P, P, 1, 16, 16, 128, None) == _lib.EINVAL
    assert f(P, P, P, P, P, 1, 0, 16, 128, None) == _lib.EINVAL
    assert f(P, P, P, P, P, 4, 16, 16, 128, None) == _lib.EINVAL
    assert f(P, P, P, P, P, 1, 16, 16, 100, None) == _lib.ESHAPE
    assert f(P + 8, P, P, P, P, 1, 16, 16, 128, None) == _lib.EALIGN
    assert f(P, P, P + 8, P, P, 1, 16, 16, 128, None) == _lib.EALIGN
    assert f(P, P, P, P, P + 2, 1, 16, 16, 128, None) == _lib.EALIGN
    assert f(P, P, P, P, P, 1, 1 << 40, 16, 128, None) == _lib.ERANGE


def test_block_gemm_split_validation(lib):
    f = lib.fp8_block_gemm_split
    assert f(None, P, P, P, P, 1, 16, 16, 128, 0, P, 1024, None) == _lib.EINVAL
    assert f(P, P, P, P, P, 1, 16, 0, 128, 0, P, 1024, None) == _lib.EINVAL
    assert f(P, P, P, P, P, 1, 16, 16, 128, 2, P, 1024, None) == _lib.EINVAL      # scale_fmt
    assert f(P, P, P, P, P, 1, 16, 16, 100, 0, P, 1024, None) == _lib.ESHAPE
    assert f(P, P, P, P, P, 1, 16, 16, 128, 0, P + 16, 1024, None) == _lib.EALIGN  # workspace
    assert f(P + 8, P, P, P, P, 1, 16, 16, 128, 1, P, 1024, None) == _lib.EALIGN
    assert f(P, P, P, P, P, 1, 1 << 40, 16, 128, 0, P, 1024, None) == _lib.ERANGE
    # sizes the GEMM would reject need no workspace (answered before any HIP call)
    assert lib.fp8_block_gemm_split_workspace(0, 16, 128) == 0
    assert lib.fp8_block_gemm_split_workspace(16, 16, 100) == 0
    assert lib.fp8_block_gemm_split_workspace(1 << 40, 16, 128) == 0


def test_weight_quant_validation(lib):
    f = lib.fp8_weight_quant
    assert f(None, 1, 8, 8, 128, 0, P, P, None) == _lib.EINVAL
    assert f(P, 1, 8, 8, 128, 0, None, P, None) == _lib.EINVAL
    assert f(P, 1, 8, 8, 128, 0, P, None, None) == _lib.EINVAL
    assert f(P, 1, 0, 8, 128, 0, P, P, None) == _lib.EINVAL
    assert f(P, 1, 8, -1, 128, 0, P, P, None) == _lib.EINVAL
    assert f(P, 2, 8, 8, 128, 0, P, P, None) == _lib.EINVAL
    assert f(P, 1, 8, 8, 128, 3, P, P, None) == _lib.EINVAL
    assert f(P, 1, 8, 8, 64, 0, P, P, None) == _lib.EUNSUPPORTED
    assert f(P + 1, 1, 8, 8, 128, 0, P, P, None) == _lib.EALIGN
    assert f(P + 2, 0, 8, 8, 128, 0, P, P, None) == _lib.EALIGN
    assert f(P, 1, 8, 8, 128, 0, P, P + 2, None) == _lib.EALIGN
    assert f(P, 1, 1 << 31, 8, 128, 0, P, P, None) == _lib.ERANGE
    assert f(P, 1, 65536 * 128, 8, 128, 0, P, P, None) == _lib.ERANGE


def test_act_quant_gemm_validation(lib):
    f = lib.fp8_act_quant_gemm
    ok = (P, 1, 0, P, P, None, P, 1, 4, 256, 512, P, P, None)

    def call(**kw):
        args = list(ok)
        for i, v in kw.items():
            args[int(i[1:])] = v
        return f(*args)

    assert call(a0=None) == _lib.EINVAL
    assert call(a3=None) == _lib.EINVAL
    assert call(a11=None) == _lib.EINVAL
    assert call(a12=None) == _lib.EINVAL
    assert call(a8=0) == _lib.EINVAL
    assert call(a1=5) == _lib.EINVAL
    assert call(a2=2) == _lib.EINVAL
    assert call(a7=9) == _lib.EINVAL
    assert call(a10=200) == _lib.ESHAPE
    assert call(a0=P + 8) == _lib.EALIGN
    assert call(a3=P + 8) == _lib.EALIGN
    assert call(a11=P + 8) == _lib.EALIGN
    assert call(a12=P + 2) == _lib.EALIGN
    assert call(a5=P + 1) == _lib.EALIGN          # bf16 bias must be 2-byte aligned
    assert call(a8=1 << 40) == _lib.ERANGE
