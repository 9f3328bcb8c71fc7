"""The C ABI from a plain C program (tests/abi_client.c): no Python or PyTorch
in the process that calls the library.

The client is compiled with gcc against include/fp8bsq.h and the in-tree
libfp8bsq.so, given seeded inputs written as raw files, and run as a child
process.  Its outputs must match the oracle: act_quant codes and scales and
weight_dequant bit for bit, the GEMMs within the oracle bound.  It also checks
on its own that invalid arguments return the documented status codes.
Cases: a decode-sized batch (M = 2: one fused kernel for act_quant_gemm) and a
tiled one (M = 300) with ragged N.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_quant_amd import _lib
from inputs import gen
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = "/opt/rocm"


@pytest.fixture(scope="module")
def client(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    lib_dir = os.path.dirname(_lib.LIB_PATH)
    if not os.path.exists(_lib.LIB_PATH):
        raise RuntimeError("libfp8bsq.so is not built")
    exe = str(tmp_path_factory.mktemp("c_client") / "abi_client")
    cmd = [gcc, "-std=c99", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", f"{ROCM}/include",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_client.c"),
           "-L", lib_dir, "-lfp8bsq", "-L", f"{ROCM}/lib", "-lamdhip64",
           f"-Wl,-rpath,{lib_dir}:{ROCM}/lib", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("m,n,k", [(2, 700, 1024), (300, 520, 2048)])
def test_c_client_matches_oracle(client, tmp_path, m, n, k):
    G.announce(f"C client m={m} n={n} k={k}")
    d = gen.custom_gemm(seed=4000 + m, m=m, n=n, k=k, outliers=True)
    x = d["x"]                                                # bf16 CPU tensor
    (tmp_path / "x.bf16").write_bytes(x.view(torch.int16).numpy().tobytes())
    (tmp_path / "w.e4m3").write_bytes(d["w"].tobytes())
    (tmp_path / "ws.f32").write_bytes(d["w_s"].tobytes())
    r = subprocess.run([client, str(tmp_path), str(m), str(n), str(k)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
    rd = lambda name, dt, shape: np.fromfile(tmp_path / name, dtype=dt).reshape(shape)
    nkb = k // 128
    xf = x.float().numpy()

    aq, as_ = oracle.act_quant(xf, 128, None)
    assert np.array_equal(rd("aq.e4m3", np.uint8, (m, k)), aq)
    assert np.array_equal(rd("as.f32", np.uint32, (m, nkb)), as_.view(np.uint32))
    ref = oracle.fp8_gemm(aq, as_, d["w"], d["w_s"])
    tol = oracle.gemm_tolerance(aq, as_, d["w"], d["w_s"])
    assert oracle.gemm_check(_bf16_to_f64(rd("c.bf16", np.uint16, (m, n))), ref, tol, "bf16").all()

    want_wd = oracle.weight_dequant(d["w"], d["w_s"], 128, "bf16")
    assert np.array_equal(rd("wd.bf16", np.uint16, (n, k)), want_wd)

    aq2, as2 = oracle.act_quant(xf, 128, "ue8m0")
    assert np.array_equal(rd("aq2.e4m3", np.uint8, (m, k)), aq2)
    assert np.array_equal(rd("as2.f32", np.uint32, (m, nkb)), as2.view(np.uint32))
    ref2 = oracle.fp8_gemm(aq2, as2, d["w"], d["w_s"])
    tol2 = oracle.gemm_tolerance(aq2, as2, d["w"], d["w_s"])
    assert oracle.gemm_check(rd("c2.f32", np.float32, (m, n)).astype(np.float64), ref2, tol2, "f32").all()
