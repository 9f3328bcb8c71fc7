"""The C ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer, on
the CPU.

abi.cpp is compiled with g++ (host code only) together with
tests/abi_host_stub.cpp, which stands in for the kernel launchers and records
each call.  tests/test_abi.py then runs in a child process against that
library, with libasan preloaded: every argument-validation check, plus the
dispatch checks that only the stub build can answer (which launcher each entry
point calls, with which arguments, and how a launch error maps to a status).
Any sanitizer report fails the child, and so this test.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp8_block_scaled_quant_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"

SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]

# Runs tests/test_abi.py with the package's __init__ (which imports torch) kept
# out of the sanitized process: only its _lib module is loaded.
RUNNER = r"""
import os, sys, types
root = sys.argv[1]
sys.path.insert(0, root)
pkg = types.ModuleType("fp8_block_scaled_quant_amd")
pkg.__path__ = [os.path.join(root, "fp8_block_scaled_quant_amd")]
sys.modules["fp8_block_scaled_quant_amd"] = pkg
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "-rs", os.path.join(root, "tests", "test_abi.py")]))
"""


def _tool(name):
    path = shutil.which(name)
    if path is None:
        pytest.skip(f"{name} not found")
    return path


@pytest.fixture(scope="module")
def stub_lib(tmp_path_factory):
    gxx = _tool("g++")
    if not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("HIP headers not found")
    out = str(tmp_path_factory.mktemp("abi_asan") / "libfp8bsq_hoststub.so")
    cmd = [gxx, "-std=c++17", "-O1", "-g", *SANITIZE, "-fPIC", "-shared", "-fvisibility=hidden",
           "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "abi.cpp"), os.path.join(ROOT, "tests", "abi_host_stub.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return out


def test_abi_under_asan_and_ubsan(stub_lib):
    asan = subprocess.run([_tool("g++"), "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("libasan not found")
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": asan,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "FP8BSQ_TEST_LIB": stub_lib,
    })
    r = subprocess.run([sys.executable, "-c", RUNNER, ROOT], capture_output=True, text=True, env=env,
                       timeout=600)
    text = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in text, text
    assert "runtime error:" not in text, text
    assert r.returncode == 0, text
    # the dispatch checks ran (they skip against the real library)
    assert "skipped" not in r.stdout.splitlines()[-1], text
