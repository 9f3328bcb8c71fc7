"""C-ABI checks that need no GPU: the library loads, exports exactly the
symbols include/fp8bsq.h declares, and rejects bad arguments with the
documented status codes before touching HIP (no kernel is launched here; the
pointers passed are never dereferenced because validation fails first).

With FP8BSQ_TEST_LIB naming the host-stub build of the ABI layer (abi.cpp
over tests/abi_host_stub.cpp, made by test_abi_sanitized.py under
AddressSanitizer and UndefinedBehaviorSanitizer), the same checks run against
it, and so do the dispatch checks at the end, which call every entry point with
valid arguments and read back which launcher the stub saw, with what."""

import ctypes
import os
import re
import subprocess

import pytest

from fp8_block_scaled_quant_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bsq.h")
LIB_PATH = os.environ.get("FP8BSQ_TEST_LIB") or _lib.LIB_PATH


def declared_symbols():
    text = open(HEADER).read()
    return set(re.findall(r"^FP8BSQ_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M))


@pytest.fixture(scope="module")
def lib():
    return _lib.load_library(None if LIB_PATH == _lib.LIB_PATH else LIB_PATH)


def test_header_declares_entry_points():
    assert declared_symbols() == set(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True)
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
                      ("FP8BSQ_ESCRATCH", _lib.ESCRATCH),
                      ("FP8BSQ_F32", _lib.F32), ("FP8BSQ_BF16", _lib.BF16),
                      ("FP8BSQ_SCALE_NONE", _lib.SCALE_NONE), ("FP8BSQ_SCALE_UE8M0", _lib.SCALE_UE8M0)]:
        assert re.search(rf"\b{name}\s*=\s*{val}\b", text), name


def test_strerror_and_version(lib):
    for st in range(8):
        assert lib.fp8bsq_strerror(st)
    assert lib.fp8bsq_strerror(99) == b"unknown status"
    assert re.match(rb"^\d+\.\d+\.\d+$", lib.fp8bsq_version())


P = 4096  # a fake, 4096-aligned non-null address: never dereferenced (validation fails first)


def test_act_quant_validation(lib):
    f = lib.fp8_act_quant
    assert f(None, 1, 8, 256, 128, 0, P, P, None) == _lib.EINVAL
    assert f(P, 1, 8, 256, 128, 0, None, P, None) == _lib.EINVAL
    assert f(P, 1, -1, 256, 128, 0, P, P, None) == _lib.EINVAL
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
    assert f(P, P, -1, 8, 128, P, 1, None) == _lib.EINVAL
    assert f(P, P, 8, 8, 128, P, 3, None) == _lib.EINVAL
    assert f(P, P, 8, 8, 256, P, 1, None) == _lib.EUNSUPPORTED
    assert f(P, P + 2, 8, 8, 128, P, 1, None) == _lib.EALIGN
    assert f(P, P, 8, 8, 128, P + 2, 0, None) == _lib.EALIGN
    assert f(P, P, 1 << 31, 8, 128, P, 1, None) == _lib.ERANGE


@pytest.mark.parametrize("name", ["fp8_block_gemm", "fp8_block_gemm_ue8m0", "fp8_block_gemm_reference"])
def test_block_gemm_validation(lib, name):
    f = getattr(lib, name)
    assert f(None, P, P, P, P, 1, 16, 16, 128, None) == _lib.EINVAL
    assert f(P, P, P, P, P, 1, -1, 16, 128, None) == _lib.EINVAL
    assert f(P, P, P, P, P, 1, 16, 16, 0, None) == _lib.EINVAL          # a product needs K
    assert f(P, P, P, P, P, 4, 16, 16, 128, None) == _lib.EINVAL
    assert f(P, P, P, P, P, 1, 16, 16, 100, None) == _lib.ESHAPE
    assert f(P + 8, P, P, P, P, 1, 16, 16, 128, None) == _lib.EALIGN
    assert f(P, P, P + 8, P, P, 1, 16, 16, 128, None) == _lib.EALIGN
    assert f(P, P, P, P, P + 2, 1, 16, 16, 128, None) == _lib.EALIGN
    assert f(P, P, P, P, P, 1, 1 << 40, 16, 128, None) == _lib.ERANGE


def test_block_gemm_split_validation(lib):
    f = lib.fp8_block_gemm_split
    assert f(None, P, P, P, P, 1, 16, 16, 128, 0, P, 1024, None) == _lib.EINVAL
    assert f(P, P, P, P, P, 1, 16, -1, 128, 0, P, 1024, None) == _lib.EINVAL
    assert f(P, P, P, P, P, 1, 16, 16, 128, 2, P, 1024, None) == _lib.EINVAL      # scale_fmt
    assert f(P, P, P, P, P, 1, 16, 16, 100, 0, P, 1024, None) == _lib.ESHAPE
    assert f(P, P, P, P, P, 1, 16, 16, 128, 0, P + 16, 1024, None) == _lib.EALIGN  # workspace
    assert f(P + 8, P, P, P, P, 1, 16, 16, 128, 1, P, 1024, None) == _lib.EALIGN
    assert f(P, P, P, P, P, 1, 1 << 40, 16, 128, 0, P, 1024, None) == _lib.ERANGE
    # sizes the GEMM would reject need no workspace (answered before any HIP call)
    assert lib.fp8_block_gemm_split_workspace(0, 16, 128) == 0
    assert lib.fp8_block_gemm_split_workspace(16, 16, 100) == 0
    assert lib.fp8_block_gemm_split_workspace(1 << 40, 16, 128) == 0


def test_block_gemm_split_noalloc_validation(lib):
    f = lib.fp8_block_gemm_split_noalloc
    assert f(None, P, P, P, P, 1, 16, 16, 128, 0, None) == _lib.EINVAL
    assert f(P, P, P, P, P, 1, 16, -1, 128, 0, None) == _lib.EINVAL
    assert f(P, P, P, P, P, 3, 16, 16, 128, 0, None) == _lib.EINVAL
    assert f(P, P, P, P, P, 1, 16, 16, 128, 2, None) == _lib.EINVAL      # scale_fmt
    assert f(P, P, P, P, P, 1, 16, 16, 100, 0, None) == _lib.ESHAPE
    assert f(P + 8, P, P, P, P, 1, 16, 16, 128, 1, None) == _lib.EALIGN
    assert f(P, P, P, P, P + 2, 1, 16, 16, 128, 1, None) == _lib.EALIGN
    assert f(P, P, P, P, P, 1, 1 << 40, 16, 128, 0, None) == _lib.ERANGE
    text = open(HEADER).read()
    assert re.search(rf"#define FP8BSQ_SPLIT_SCRATCH_BYTES \(\(size_t\){_lib.SPLIT_SCRATCH_BYTES}\)", text)


def test_weight_quant_validation(lib):
    f = lib.fp8_weight_quant
    assert f(None, 1, 8, 8, 128, 0, P, P, None) == _lib.EINVAL
    assert f(P, 1, 8, 8, 128, 0, None, P, None) == _lib.EINVAL
    assert f(P, 1, 8, 8, 128, 0, P, None, None) == _lib.EINVAL
    assert f(P, 1, -1, 8, 128, 0, P, P, None) == _lib.EINVAL
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
    assert call(a8=-1) == _lib.EINVAL
    assert call(a10=0) == _lib.EINVAL                 # a product needs K
    # no weight rows: the quantizer's pointers are still checked (a launch would follow)
    assert call(a9=0, a0=None) == _lib.EINVAL
    assert call(a9=0, a12=None) == _lib.EINVAL
    assert call(a9=0, a11=P + 8) == _lib.EALIGN
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


def test_empty_inputs_return_ok_without_reading_pointers(lib):
    """A call with no output elements returns FP8BSQ_OK before any pointer
    check or HIP call (NULL pointers here; no GPU is needed), once the enum
    and shape checks have passed."""
    N = None
    assert lib.fp8_act_quant(N, 1, 0, 256, 128, 0, N, N, N) == _lib.OK
    assert lib.fp8_act_quant(N, 1, 8, 0, 128, 1, N, N, N) == _lib.OK
    assert lib.fp8_act_quant(N, 1, 0, 200, 128, 0, N, N, N) == _lib.ESHAPE
    assert lib.fp8_act_quant(N, 9, 0, 256, 128, 0, N, N, N) == _lib.EINVAL
    assert lib.fp8_act_quant(N, 1, 0, 256, 64, 0, N, N, N) == _lib.EUNSUPPORTED
    for f in (lib.fp8_weight_dequant,):
        assert f(N, N, 0, 300, 128, N, 1, N) == _lib.OK
        assert f(N, N, 300, 0, 128, N, 0, N) == _lib.OK
        assert f(N, N, 0, 300, 128, N, 5, N) == _lib.EINVAL
    assert lib.fp8_weight_quant(N, 1, 0, 300, 128, 1, N, N, N) == _lib.OK
    assert lib.fp8_weight_quant(N, 0, 300, 0, 128, 0, N, N, N) == _lib.OK
    assert lib.fp8_weight_quant(N, 0, 0, 300, 128, 4, N, N, N) == _lib.EINVAL
    for name in ("fp8_block_gemm", "fp8_block_gemm_ue8m0", "fp8_block_gemm_reference"):
        f = getattr(lib, name)
        assert f(N, N, N, N, N, 1, 0, 256, 512, N) == _lib.OK, name
        assert f(N, N, N, N, N, 0, 16, 0, 512, N) == _lib.OK, name
        assert f(N, N, N, N, N, 1, 0, 256, 0, N) == _lib.EINVAL, name
        assert f(N, N, N, N, N, 1, 0, 256, 100, N) == _lib.ESHAPE, name
    assert lib.fp8_block_gemm_split(N, N, N, N, N, 1, 0, 256, 512, 1, N, 0, N) == _lib.OK
    assert lib.fp8_block_gemm_split(N, N, N, N, N, 1, 16, 0, 512, 0, N, 0, N) == _lib.OK
    assert lib.fp8_block_gemm_split(N, N, N, N, N, 1, 0, 256, 512, 3, N, 0, N) == _lib.EINVAL
    assert lib.fp8_block_gemm_split_noalloc(N, N, N, N, N, 1, 0, 256, 512, 1, N) == _lib.OK
    assert lib.fp8_block_gemm_split_noalloc(N, N, N, N, N, 0, 16, 0, 512, 0, N) == _lib.OK
    assert lib.fp8_block_gemm_split_workspace(0, 256, 512) == 0
    assert lib.fp8_act_quant_gemm(N, 1, 0, N, N, N, N, 1, 0, 256, 512, N, N, N) == _lib.OK
    assert lib.fp8_act_quant_gemm(N, 1, 0, N, N, N, N, 1, 0, 0, 512, N, N, N) == _lib.OK
    assert lib.fp8_act_quant_gemm(N, 1, 0, N, N, N, N, 1, 0, 256, 0, N, N, N) == _lib.EINVAL


# ------------------------------------------------ dispatch (host-stub build only)

class Stub:
    def __init__(self, lib):
        if not hasattr(lib, "_fp8bsq_stub_last"):
            pytest.skip("dispatch checks need the host-stub build (test_abi_sanitized.py)")
        self.lib = lib
        lib._fp8bsq_stub_last.restype = ctypes.c_int
        lib._fp8bsq_stub_last.argtypes = [ctypes.c_char_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(ctypes.c_void_p)]

    def last(self):
        name = ctypes.create_string_buffer(64)
        ints = (ctypes.c_int64 * 16)()
        ptrs = (ctypes.c_void_p * 12)()
        n = self.lib._fp8bsq_stub_last(name, 64, ints, ptrs)
        return n, name.value.decode(), list(ints), [p or 0 for p in ptrs]


def test_dispatch_quantizers(lib):
    st = Stub(lib)
    S = 0x7000
    assert lib.fp8_act_quant(P, 1, 8, 256, 128, 1, P + 16, P + 32, S) == _lib.OK
    _, name, ints, ptrs = st.last()
    assert name == "act_quant" and ints[:3] == [1, 16, 1] and ptrs[:4] == [P, P + 16, P + 32, S]
    assert lib.fp8_act_quant(P, 0, 3, 384, 128, 0, P, P, None) == _lib.OK
    assert st.last()[2][:3] == [0, 9, 0]
    assert lib.fp8_weight_dequant(P + 1, P, 300, 130, 128, P + 2, 1, S) == _lib.OK
    _, name, ints, ptrs = st.last()
    assert name == "weight_dequant" and ints[:3] == [300, 130, 1] and ptrs[:4] == [P + 1, P, P + 2, S]
    assert lib.fp8_weight_quant(P, 1, 300, 130, 128, 1, P + 8, P + 4, S) == _lib.OK
    _, name, ints, ptrs = st.last()
    assert name == "weight_quant" and ints[:4] == [1, 300, 130, 1] and ptrs[:4] == [P, P + 8, P + 4, S]


def test_dispatch_gemms(lib):
    st = Stub(lib)
    S = 0x7000
    a, a_s, b, b_s, c = P, P + 0x100, P + 0x200, P + 0x300, P + 0x400
    for fn, name, pow2 in [("fp8_block_gemm", "block_gemm", 0), ("fp8_block_gemm_ue8m0", "block_gemm", 1),
                           ("fp8_block_gemm_reference", "block_gemm_reference", None)]:
        assert getattr(lib, fn)(a, a_s, b, b_s, c, 1, 300, 700, 1024, S) == _lib.OK
        _, got, ints, ptrs = st.last()
        assert got == name and ints[:4] == [1, 300, 700, 1024], fn
        assert ptrs[:7] == [a, a_s, b, b_s, c, S, 0], fn       # bias null
        if pow2 is not None:
            assert ints[4] == pow2, fn
    assert lib.fp8_block_gemm_split_workspace(300, 700, 1024) == 300 * 1000000 + 700 * 1000 + 1024
    assert lib.fp8_block_gemm_split(a, a_s, b, b_s, c, 0, 300, 700, 1024, 1, P + 0x1000, 5000, S) == _lib.OK
    _, got, ints, ptrs = st.last()
    assert got == "block_gemm_split" and ints[:6] == [0, 300, 700, 1024, 1, 5000]
    assert ptrs[:7] == [a, a_s, b, b_s, c, S, P + 0x1000]
    assert lib.fp8_block_gemm_split(a, a_s, b, b_s, c, 0, 300, 700, 1024, 0, None, 5000, S) == _lib.OK
    assert st.last()[2][4:6] == [0, 0]                      # no workspace: zero bytes passed on


def test_dispatch_split_noalloc(lib):
    st = Stub(lib)
    S = 0x7000
    a, a_s, b, b_s, c = P, P + 0x100, P + 0x200, P + 0x300, P + 0x400
    assert lib.fp8_block_gemm_split_noalloc(a, a_s, b, b_s, c, 1, 300, 700, 1024, 1, S) == _lib.OK
    _, got, ints, ptrs = st.last()
    assert got == "block_gemm_split_noalloc" and ints[:5] == [1, 300, 700, 1024, 1]
    assert ptrs[:6] == [a, a_s, b, b_s, c, S]
    n0 = st.last()[0]
    assert lib.fp8_block_gemm_split_noalloc(a, a_s, b, b_s, c, 1, 777, 700, 1024, 0, S) == _lib.ESCRATCH
    assert st.last()[0] == n0                                 # nothing launched


def test_dispatch_act_quant_gemm(lib):
    st = Stub(lib)
    S = 0x7000
    x, b, b_s, bias, c, a_q, a_s = P, P + 0x100, P + 0x200, P + 0x300, P + 0x400, P + 0x500, P + 0x600
    n0 = st.last()[0]
    assert lib.fp8_act_quant_gemm(x, 1, 1, b, b_s, bias, c, 1, 2, 256, 512, a_q, a_s, S) == _lib.OK
    n1, name, ints, ptrs = st.last()
    assert n1 == n0 + 1 and name == "act_quant_gemm_fused"
    assert ints[:5] == [1, 1, 2, 256, 512] and ptrs[:8] == [x, b, b_s, bias, c, a_q, a_s, S]
    assert lib.fp8_act_quant_gemm(x, 1, 0, b, b_s, None, c, 0, 40, 256, 512, a_q, a_s, S) == _lib.OK
    n2, name, ints, ptrs = st.last()
    assert n2 == n1 + 2 and name == "block_gemm"           # act_quant, then the GEMM
    assert ints[:5] == [0, 40, 256, 512, 0] and ptrs[:7] == [a_q, a_s, b, b_s, c, S, 0]
    # no weight rows: act_quant alone, with b, b_s and c never read
    assert lib.fp8_act_quant_gemm(x, 1, 1, None, None, None, None, 1, 40, 0, 512, a_q, a_s, S) == _lib.OK
    n3, name, ints, ptrs = st.last()
    assert n3 == n2 + 1 and name == "act_quant"
    assert ints[:3] == [1, 160, 1] and ptrs[:4] == [x, a_q, a_s, S]
    # empty calls launch nothing
    for args in [(x, 1, 0, b, b_s, None, c, 1, 0, 256, 512, a_q, a_s, S)]:
        assert lib.fp8_act_quant_gemm(*args) == _lib.OK
    assert lib.fp8_block_gemm(None, None, None, None, None, 1, 0, 256, 512, S) == _lib.OK
    assert lib.fp8_act_quant(None, 1, 0, 256, 128, 0, None, None, S) == _lib.OK
    assert lib.fp8_weight_dequant(None, None, 0, 256, 128, None, 1, S) == _lib.OK
    assert st.last()[0] == n3


def test_launch_error_maps_to_elaunch(lib):
    Stub(lib)
    lib._fp8bsq_stub_fail_next.restype = None
    lib._fp8bsq_stub_fail_next()
    assert lib.fp8_act_quant(P, 1, 8, 256, 128, 0, P, P, None) == _lib.ELAUNCH
    assert lib.fp8_act_quant(P, 1, 8, 256, 128, 0, P, P, None) == _lib.OK
    lib._fp8bsq_stub_fail_next()
    assert lib.fp8_act_quant_gemm(P, 1, 0, P, P, None, P, 1, 40, 256, 512, P, P, None) == _lib.ELAUNCH
