"""The quantizers and the dequantizer at their largest sizes.

* act_quant of bf16 activations past 4 GiB ([300000, 7168], 4.3 GB: rows
  from 299,593 on lie past byte 2^32), both scale formats;
* weight_dequant of a weight past 4 GiB ([599187, 7168] codes, 8.6 GB of bf16
  out);
* weight_dequant with 65,536 tile rows, one past the tile kernel's grid limit,
  which takes the element-wise kernel; and weight_quant at its own limit,
  65,535 tile rows (one more is FP8BSQ_ERANGE, checked on the CPU).

All calls go through the C ABI.  Results are checked bit for bit against the
oracle on sampled rows (or 128-row bands for weight_quant): the first and
last, those around byte 2^32 of the large operand, and seeded random ones.
The large inputs come from the seeded chunked generators.
"""

import ctypes
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_quant_amd import _lib
from inputs import gen
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

K = 7168
CHUNK = 16384


def _rows(n: int, seed: int, extra=()) -> np.ndarray:
    rng = np.random.default_rng(seed)
    s = {0, 1, 127, 128, n - 2, n - 1, *extra}
    s |= set(rng.choice(n, 200, replace=False).tolist())
    return np.array(sorted(r for r in s if 0 <= r < n))


def test_act_quant_past_4gib():
    m = 300000
    edge = (1 << 32) // (2 * K)                      # first row with bytes past 2^32
    rows = _rows(m, 3, (edge - 1, edge, edge + 1))
    G.announce(f"act_quant bf16 [{m}, {K}] ({2 * m * K / 2**30:.2f} GiB), chunks built in parallel")
    dev = G.device()
    x = torch.empty((m, K), dtype=torch.bfloat16, device=dev)
    kept = np.empty((len(rows), K), dtype=np.float32)
    nchunks = -(-m // CHUNK)
    with ThreadPoolExecutor(8) as ex:
        for i, c in enumerate(ex.map(lambda j: gen.activations_chunk(31, m, K, j, CHUNK), range(nchunks))):
            r0 = i * CHUNK
            x[r0:r0 + c.shape[0]].copy_(c)
            sel = np.nonzero((rows >= r0) & (rows < r0 + c.shape[0]))[0]
            kept[sel] = c[torch.from_numpy(rows[sel] - r0)].float().numpy()
    torch.cuda.synchronize()
    lib = _lib.lib()
    y = G.Guarded(m * K)
    s = G.Guarded(m * (K // 128) * 4)
    for fmt, code in ((None, _lib.SCALE_NONE), ("ue8m0", _lib.SCALE_UE8M0)):
        st = lib.fp8_act_quant(ctypes.c_void_p(x.data_ptr()), _lib.BF16, m, K, 128, code,
                               ctypes.c_void_p(y.ptr), ctypes.c_void_p(s.ptr), G.stream())
        assert st == _lib.OK, st
        torch.cuda.synchronize()
        y.check_guards()
        s.check_guards()
        idx = torch.from_numpy(rows).to(dev)
        codes = y.payload().view(m, K)[idx].cpu().numpy()
        scales = s.payload().view(torch.float32).view(m, K // 128)[idx].cpu().numpy()
        wq, ws = oracle.act_quant(kept, 128, fmt)
        assert np.array_equal(codes, wq), f"scale_fmt={fmt}: codes differ on {int((codes != wq).any(1).sum())} rows"
        assert np.array_equal(scales.view(np.uint32), ws.view(np.uint32)), f"scale_fmt={fmt}: scales differ"


def _dequant_rows_check(y_dev, m, n, rows, kept, s_host):
    got = y_dev.view(torch.int16).view(m, n)[torch.from_numpy(rows).to(y_dev.device)].cpu().numpy().view(np.uint16)
    for i, r in enumerate(rows):
        want = oracle.weight_dequant(kept[i][None, :], s_host[r // 128][None, :], 128, "bf16")[0]
        assert np.array_equal(got[i], want), f"row {r}: {int((got[i] != want).sum())} elements differ"


def test_weight_dequant_past_4gib():
    n_rows = (1 << 32) // K + 1                        # 599187: the last row straddles byte 2^32
    rows = _rows(n_rows, 4, (n_rows - 3,))
    G.announce(f"weight_dequant [{n_rows}, {K}] -> bf16 ({3 * n_rows * K / 2**30:.1f} GiB moved)")
    dev = G.device()
    x = torch.empty((n_rows, K), dtype=torch.uint8, device=dev)
    kept = np.empty((len(rows), K), dtype=np.uint8)
    for r0, c in gen.weight_codes_chunks(41, n_rows, K):
        x[r0:r0 + c.shape[0]].copy_(torch.from_numpy(c))
        sel = np.nonzero((rows >= r0) & (rows < r0 + c.shape[0]))[0]
        kept[sel] = c[rows[sel] - r0]
    s_host = gen.log_uniform_scales(gen.rng_for(42), gen.scale_grid(n_rows, K), -14, -2)
    s_dev = torch.from_numpy(s_host).to(dev)
    y = G.Guarded(n_rows * K * 2)
    st = _lib.lib().fp8_weight_dequant(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(s_dev.data_ptr()),
                                       n_rows, K, 128, ctypes.c_void_p(y.ptr), _lib.BF16, G.stream())
    assert st == _lib.OK, st
    torch.cuda.synchronize()
    y.check_guards()
    _dequant_rows_check(y.payload(), n_rows, K, rows, kept, s_host)


def test_weight_dequant_past_the_tile_grid():
    """65,536 tile rows: one past grid.y's limit, so the element-wise kernel runs."""
    n_rows, n = 65535 * 128 + 1, 16
    rows = _rows(n_rows, 5, (65535 * 128 - 1,))
    G.announce(f"weight_dequant [{n_rows}, {n}] (element-wise kernel)")
    dev = G.device()
    codes = gen.weight_codes(gen.rng_for(51), n_rows, n)
    s_host = gen.log_uniform_scales(gen.rng_for(52), gen.scale_grid(n_rows, n), -14, -2)
    x = torch.from_numpy(codes).to(dev)
    s_dev = torch.from_numpy(s_host).to(dev)
    y = G.Guarded(n_rows * n * 2)
    st = _lib.lib().fp8_weight_dequant(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(s_dev.data_ptr()),
                                       n_rows, n, 128, ctypes.c_void_p(y.ptr), _lib.BF16, G.stream())
    assert st == _lib.OK, st
    torch.cuda.synchronize()
    y.check_guards()
    _dequant_rows_check(y.payload(), n_rows, n, rows, codes[rows], s_host)


def test_weight_quant_at_the_tile_grid_limit():
    """65,535 tile rows, the most the tile kernel's grid takes."""
    n_rows, n = 65535 * 128, 16
    G.announce(f"weight_quant bf16 [{n_rows}, {n}]")
    dev = G.device()
    w = gen.activations(gen.rng_for(61), n_rows, n)           # bf16 N(0, 1)
    wd = w.to(dev)
    y = G.Guarded(n_rows * n)
    s = G.Guarded(65535 * 4)
    st = _lib.lib().fp8_weight_quant(ctypes.c_void_p(wd.data_ptr()), _lib.BF16, n_rows, n, 128,
                                     _lib.SCALE_UE8M0, ctypes.c_void_p(y.ptr), ctypes.c_void_p(s.ptr),
                                     G.stream())
    assert st == _lib.OK, st
    torch.cuda.synchronize()
    y.check_guards()
    s.check_guards()
    codes = y.payload().view(n_rows, n)
    scales = s.payload().view(torch.float32).cpu().numpy()
    bands = _rows(65535, 6)
    wf = w.float().numpy()
    for t in bands:
        want_q, want_s = oracle.weight_quant(wf[128 * t:128 * (t + 1)], 128, "ue8m0")
        got_q = codes[128 * t:128 * (t + 1)].cpu().numpy()
        assert np.array_equal(got_q, want_q), f"tile row {t}: codes differ"
        assert scales[t:t + 1].view(np.uint32)[0] == want_s.view(np.uint32)[0, 0], f"tile row {t}: scale differs"
