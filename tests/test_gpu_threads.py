"""Concurrent callers: the C ABI's calls are re-entrant and thread-safe.

Four host threads, each with its own stream and its own inputs, call
act_quant, the GEMM (split-K allowed, with its workspace from torch's
allocator), weight_dequant and act_quant_gemm over and over, with ctypes
releasing the interpreter lock inside every library call.  Every result must be
bit-identical to the same call made alone on the default stream beforehand (the
kernels are deterministic).  The allocation-free split entry point shares one
scratch array per GPU and is documented as racing under overlap; it is not
used here.
"""

import threading

import pytest
import torch

import fp8_block_scaled_quant_amd as fb
from inputs import gen
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

SHAPES = [(1, 2304, 7168), (40, 1000, 1024), (300, 700, 2048), (512, 1024, 8192)]


def _run(x, w, ws):
    y, s = fb.act_quant(x, 128, "ue8m0")
    c = fb.fp8_gemm(y, s, w, ws, torch.bfloat16, "ue8m0")
    deq = fb.weight_dequant(w, ws, 128, torch.bfloat16)
    c2, y2, s2 = fb.act_quant_gemm(x, w, ws)
    return y.view(torch.uint8), s, c, deq, c2, y2.view(torch.uint8), s2


def test_threads_on_their_own_streams_match_serial_results():
    dev = G.device()
    G.announce(f"4 threads x {len(SHAPES)} shapes, own streams")
    inputs = []
    for i, (m, n, k) in enumerate(SHAPES):
        d = gen.custom_gemm(seed=600 + i, m=m, n=n, k=k)
        inputs.append((d["x"].to(dev), torch.from_numpy(d["w"]).to(dev), torch.from_numpy(d["w_s"]).to(dev)))
    expect = [_run(*inp) for inp in inputs]
    torch.cuda.synchronize()

    errors = []

    def worker(t):
        try:
            stream = torch.cuda.Stream(device=dev)
            with torch.cuda.stream(stream):
                for it in range(12):
                    i = (t + it) % len(inputs)
                    got = _run(*inputs[i])
                    stream.synchronize()
                    for a, b in zip(got, expect[i]):
                        if not torch.equal(a, b):
                            errors.append(f"thread {t} iteration {it} shape {SHAPES[i]}")
                            return
        except Exception as e:      # reported below, in the test's own thread
            errors.append(f"thread {t}: {e!r}")

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
