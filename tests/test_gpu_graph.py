"""HIP graph capture of the quantize-and-multiply path.

No entry point allocates, synchronizes or issues a memset (split-K clears
its counters with a kernel), so a step made of them captures into a graph
(torch.cuda.graph): the decode case, where one step is ~25 us of kernel time
and launch overhead matters, a tiled one, and a split-K one (its workspace
from torch's graph pool).
Each case replays the graph on several fresh inputs copied into the captured
input buffer, with eager work and synchronizations between replays, and
checks every replay bit for bit against the same calls made eagerly.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as fb
from inputs import gen
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


# M = 1 and 8: act_quant fused into the decode GEMM (one kernel, helper waves
# and LDS counters); M = 12: the same through the LDS ring; M = 20: act_quant
# then the decode GEMM; M = 300: act_quant then the tiled GEMM.
@pytest.mark.parametrize("m,n,k,scale_fmt", [(1, 18432, 7168, None), (8, 18432, 7168, None),
                                             (12, 18432, 7168, None), (20, 18432, 7168, None),
                                             (300, 2304, 1024, "ue8m0")])
def test_step_replays_match_eager(m, n, k, scale_fmt):
    dev = G.device()
    G.announce(f"graph capture m={m} n={n} k={k} scale_fmt={scale_fmt}")
    d = gen.custom_gemm(seed=500 + m, m=m, n=n, k=k)
    w = torch.from_numpy(d["w"]).to(dev)
    ws = torch.from_numpy(d["w_s"]).to(dev)
    rng = np.random.default_rng(600 + m)
    inputs = [gen.activations(rng, m, k).to(dev) for _ in range(3)]

    def step(x):
        c_fused, y, s = fb.act_quant_gemm(x, w, ws, scale_fmt)
        y2, s2 = fb.act_quant(x, 128, scale_fmt)
        c_two = fb.fp8_gemm(y2, s2, w, ws, torch.bfloat16, scale_fmt)
        return c_fused, y, s, c_two

    static_x = inputs[0].clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(static_x)                       # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = step(static_x)

    for i, x in enumerate(inputs):
        static_x.copy_(x)
        graph.replay()
        torch.cuda.synchronize()
        eager = step(x)
        torch.cuda.synchronize()
        for name, got, ref in zip(("act_quant_gemm", "codes", "scales", "act_quant + fp8_gemm"),
                                  captured, eager):
            assert torch.equal(got.view(torch.uint8) if got.dtype == torch.float8_e4m3fn else got,
                               ref.view(torch.uint8) if ref.dtype == torch.float8_e4m3fn else ref), \
                f"replay {i}: {name} differs from the eager call"
        # the fused call and the two-call path agree as well
        assert torch.equal(captured[0], captured[3]), f"replay {i}: fused and two-call outputs differ"


def test_split_k_replays_match_eager():
    """fp8_gemm with a split-K tail (8 tiles in 4 parts: a counter-clearing
    launch, then partials, counters and the last part's sum) inside a graph."""
    m, n, k = 512, 1024, 8192
    dev = G.device()
    G.announce(f"graph capture split-K m={m} n={n} k={k}")
    assert fb._lib.lib().fp8_block_gemm_split_workspace(m, n, k) > 0
    d = gen.custom_gemm(seed=700, m=m, n=n, k=k)
    w = torch.from_numpy(d["w"]).to(dev)
    ws = torch.from_numpy(d["w_s"]).to(dev)
    rng = np.random.default_rng(701)
    inputs = [gen.activations(rng, m, k).to(dev) for _ in range(3)]

    def step(x):
        y, s = fb.act_quant(x, 128, "ue8m0")
        return fb.fp8_gemm(y, s, w, ws, torch.bfloat16, "ue8m0")

    static_x = inputs[0].clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(static_x)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = step(static_x)
    for i, x in enumerate(inputs):
        static_x.copy_(x)
        graph.replay()
        torch.cuda.synchronize()
        eager = step(x)
        torch.cuda.synchronize()
        assert torch.equal(captured, eager), f"replay {i} differs from the eager call"
