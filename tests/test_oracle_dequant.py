"""Pins for the oracle's weight_dequant.

* scale-grid shapes: the page's 1024x1024 -> 8x8 example; ceil-division grids
  for ragged sizes, and rejection of any other grid shape;
* special cases: s = 1 gives the code values exactly; s = 2^k gives them scaled
  by 2^k exactly; a distinct power of two per tile pins which scale each
  element uses (row block, column block, row-major order of the grid);
* general scales: bit-identical to torch's CPU fp8 decode times the scale,
  then torch's bf16 cast (round to nearest even).
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from inputs import gen
from tests.exact import torch_e4m3_table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
with open(os.path.join(GOLDEN, "page_facts.json")) as _f:
    FACTS = json.load(_f)

TABLE = torch_e4m3_table()


def check_page_grid(weight_dequant):
    ex = FACTS["scale_grid_example"]
    m, n = ex["weight_shape"]
    w = gen.weight_codes(np.random.default_rng(0), m, n)
    s = np.ones(ex["scale_shape"], np.float32)
    y = weight_dequant(w, s, ex["block_size"], "f32")
    assert y.shape == (m, n)
    with pytest.raises(ValueError):
        weight_dequant(w, np.ones((9, 8), np.float32), ex["block_size"], "f32")


def check_ragged_grid(weight_dequant):
    w = gen.weight_codes(np.random.default_rng(1), 300, 130)
    with pytest.raises(ValueError):
        weight_dequant(w, np.ones((2, 1), np.float32), 128, "f32")      # floor grid refused
    s = np.ones((3, 2), np.float32)
    assert weight_dequant(w, s, 128, "f32").shape == (300, 130)


def check_unit_and_pow2(weight_dequant):
    w = np.array([c for c in range(256) if c not in (0x7F, 0xFF)] * 2, np.uint8)[:384].reshape(3, 128)
    y = weight_dequant(w, np.ones((1, 1), np.float32), 128, "f32")
    assert np.array_equal(y.astype(np.float64), TABLE[w])
    for k in (-14, -3, 0, 5):
        y = weight_dequant(w, np.full((1, 1), 2.0**k, np.float32), 128, "f32")
        assert np.array_equal(y.astype(np.float64), np.ldexp(TABLE[w], k))


def check_tile_mapping(weight_dequant):
    m, n = 300, 520                       # ragged in both directions: grid [3, 5]
    gm, gn = 3, 5
    w = np.full((m, n), 0x38, np.uint8)   # every code is 1.0
    s = (2.0 ** np.arange(gm * gn, dtype=np.float64).reshape(gm, gn) * 2.0**-7).astype(np.float32)
    y = weight_dequant(w, s, 128, "f32")
    r = np.arange(m)[:, None] // 128
    c = np.arange(n)[None, :] // 128
    assert np.array_equal(y, (2.0 ** (r * gn + c) * 2.0**-7).astype(np.float32))
    assert y[299, 519] == s[2, 4] and y[0, 0] == s[0, 0] and y[127, 128] == s[0, 1]


def torch_dequant_bf16(w, s):
    m, n = w.shape
    full = np.repeat(np.repeat(s, 128, 0)[:m], 128, 1)[:, :n]
    t = torch.from_numpy(w).view(torch.float8_e4m3fn).float() * torch.from_numpy(full)
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16), t.numpy()


def check_vs_torch(weight_dequant, m, n, seed):
    d = gen.dequant_workload(m, n, seed=seed)
    bf, f32 = torch_dequant_bf16(d["w"], d["w_s"])
    assert np.array_equal(weight_dequant(d["w"], d["w_s"], 128, "bf16"), bf)
    assert np.array_equal(weight_dequant(d["w"], d["w_s"], 128, "f32").view(np.uint32), f32.view(np.uint32))


def test_page_grid():
    check_page_grid(oracle.weight_dequant)


def test_ragged_grid():
    check_ragged_grid(oracle.weight_dequant)


def test_unit_and_pow2_scales():
    check_unit_and_pow2(oracle.weight_dequant)


def test_tile_mapping():
    check_tile_mapping(oracle.weight_dequant)


@pytest.mark.parametrize("m,n,seed", [(256, 384, 2), (300, 520, 12), (1, 1, 3), (129, 127, 4)])
def test_vs_torch(m, n, seed):
    check_vs_torch(oracle.weight_dequant, m, n, seed)


def test_bf16_rounding_cases():
    v = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-20, -1.0 - 2**-8,
                  3.4e38, np.inf, -np.inf, 2.0**-140], np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16_bits(v), want)
    assert np.isnan(oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(np.array([np.nan], np.float32))))[0]
