"""Compile the HIP sources into the in-tree shared library ``libfp8bsq.so``.

gfx950 only.  Packed-FP32 instruction selection is switched off for every HIP
source, floating-point contraction is off unless a kernel asks for a fused
multiply-add explicitly, and no fast-math flag is used (the quantizer relies on
IEEE division and exact fused multiply-adds).
"""

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfp8bsq.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["abi.cpp", "act_quant.hip", "weight_dequant.hip", "weight_quant.hip", "block_gemm.hip"]

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libfp8bsq")
    return path


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source for gfx950 and link ``libfp8bsq.so``; returns its path."""
    objdir = os.path.join(PKG_DIR, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, *lang, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _drain(procs[:1])
            procs = procs[1:]
    _drain(procs)
    tmp = LIB_PATH + ".tmp"
    link = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), file=sys.stderr)
    out = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if out.returncode != 0:
        raise RuntimeError("link failed:\n" + out.stdout.decode(errors="replace"))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _drain(procs):
    for src, p in procs:
        text, _ = p.communicate()
        if p.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n" + text.decode(errors="replace"))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
