"""Pins for the oracle's weight_quant (128 x 128 block weight quantization).

* special case reducing to the pinned act_quant: a tile whose rows are all
  copies of one row has the row's 1 x 128 block amax, so its scale and codes
  must equal act_quant's for that row (and M = 1 is a single such row);
* exact rational arithmetic on adversarial tiles (elements on E4M3 rounding
  midpoints, and every bf16 magnitude under fixed maxima): each code is the
  E4M3 value nearest the fp32 quotient fl32(x / s), s = fl32(amax / 448);
* closed forms: an all-zero tile gets s = fl32(fl32(1e-4)/448) = 0x346FACAD
  (2^-22 under ue8m0) and codes 0, keeping the sign of -0; each tile's largest
  element encodes to +-448 (scale_fmt None) or into [224, 448] (ue8m0);
* the scale grid is [ceil(M/128), ceil(N/128)] -- the page's 1024 x 1024
  example gives 8 x 8 -- and an edge tile's scale comes from its valid
  elements alone (checked against exact rational arithmetic);
* quantize -> dequantize (through the pinned weight_dequant oracle) is within
  half an E4M3 ulp of the fp32 quotient, times the scale, plus the two fp32
  roundings (quotient and product), for every element;
* a second, independent CPU composition through torch's own ops (tile amax,
  clamp, division, frexp, fp8 cast) is bit-identical.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from inputs import gen
from tests.exact import f32_round, nearest_e4m3_bruteforce, torch_e4m3_table
from tests.test_oracle_act_quant import tiny_blocks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
with open(os.path.join(GOLDEN, "page_facts.json")) as _f:
    FACTS = json.load(_f)

CLAMP = FACTS["amax_clamp_min"]["value"]
DIV = FACTS["scale_formula"]["divisor"]
TABLE = torch_e4m3_table()


def _bits(v) -> int:
    return int(np.float32(v).view(np.uint32))


def small_weights(m=384, n=640, seed=21):
    return gen.weight_quant_workload(m, n, seed=seed)["w"].float().numpy()


# ---------------------------------------------------------------- reduction to act_quant

def check_identical_rows_match_act_quant(weight_quant, scale_fmt):
    rng = np.random.default_rng(3)
    row = gen.to_bf16(rng.standard_normal((1, 1024), dtype=np.float32) * 2).float().numpy()
    row[0, 256:384] *= 1e-7                      # one block under the clamp
    aq, as_ = oracle.act_quant(row, 128, scale_fmt)
    for m in (1, 77, 128):
        x = np.repeat(row, m, axis=0)
        q, s = weight_quant(x, 128, scale_fmt)
        assert s.shape == (1, 8)
        assert np.array_equal(s.view(np.uint32), as_.view(np.uint32))
        assert np.array_equal(q, np.repeat(aq, m, axis=0))


@pytest.mark.parametrize("scale_fmt", [None, "ue8m0"])
def test_identical_rows_match_act_quant(scale_fmt):
    check_identical_rows_match_act_quant(oracle.weight_quant, scale_fmt)


# ---------------------------------------------------------------- closed forms

def check_zero_tile(weight_quant):
    x = np.ones((256, 256), dtype=np.float32)
    x[128:, :128] = 0.0
    x[130, 5] = -0.0
    q, s = weight_quant(x, 128, None)
    want = f32_round(Fraction(float(np.float32(CLAMP))) / Fraction(DIV))
    assert _bits(s[1, 0]) == _bits(want) == 0x346FACAD
    assert np.all((q[128:, :128] & 0x7F) == 0)
    assert q[130, 5] == 0x80 and q[130, 4] == 0x00
    qu, su = weight_quant(x, 128, "ue8m0")
    assert _bits(su[1, 0]) == 0x34800000
    assert np.all((qu[128:, :128] & 0x7F) == 0)


def check_tile_max_hits_448(weight_quant):
    x = small_weights()
    x[:128, 128:256] *= np.float32(1e-8)         # a tile under the clamp (already tiny magnitudes)
    m, n = x.shape
    q, s = weight_quant(x, 128, None)
    qu, su = weight_quant(x, 128, "ue8m0")
    hits = 0
    for i in range(s.shape[0]):
        for j in range(s.shape[1]):
            blk = np.abs(x[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)])
            r, c = np.unravel_index(np.argmax(blk), blk.shape)
            top = q[128 * i + r, 128 * j + c] & 0x7F
            topu = qu[128 * i + r, 128 * j + c] & 0x7F
            if blk.max() >= np.float32(CLAMP):
                assert top == 0x7E, (i, j)
                assert 0x76 <= topu <= 0x7E, (i, j)
                hits += 1
            else:
                assert top != 0x7E
    assert hits >= s.size - 2


def test_zero_tile():
    check_zero_tile(oracle.weight_quant)


def test_tile_max_hits_448():
    check_tile_max_hits_448(oracle.weight_quant)


def check_grid_and_edge_tiles(weight_quant):
    ex = FACTS["scale_grid_example"]
    x = np.random.default_rng(0).standard_normal(ex["weight_shape"], dtype=np.float32)
    _, s = weight_quant(x, ex["block_size"], None)
    assert s.shape == tuple(ex["scale_shape"])
    # ragged: the edge tile's scale comes from its valid elements only
    x = np.random.default_rng(1).standard_normal((130, 200), dtype=np.float32)
    x[:128, :128] *= 1000.0
    q, s = weight_quant(x, 128, None)
    assert s.shape == (2, 2) and q.shape == (130, 200)
    for (i, j) in ((0, 1), (1, 0), (1, 1)):
        valid = x[128 * i:min(128 * (i + 1), 130), 128 * j:min(128 * (j + 1), 200)]
        amax = max(Fraction(float(np.max(np.abs(valid)))), Fraction(float(np.float32(CLAMP))))
        assert s[i, j] == f32_round(amax / Fraction(DIV)), (i, j)


def test_grid_and_edge_tiles():
    check_grid_and_edge_tiles(oracle.weight_quant)


def test_rejects_bad_input():
    with pytest.raises(TypeError):
        oracle.weight_quant(np.zeros((2, 2, 2), np.float32))
    with pytest.raises(ValueError):
        oracle.weight_quant(np.full((4, 4), np.inf, np.float32))
    with pytest.raises(ValueError):
        oracle.weight_quant(np.zeros((4, 4), np.float32), scale_fmt="e8m0")


# ---------------------------------------------------------------- exact quotients

def adversarial_tiles():
    """Single-tile weights whose elements sit at E4M3 rounding midpoints.

    For a tile scale s, elements fl32(mid * s) put the fp32 quotient on or one
    fp32 ulp from a midpoint between adjacent E4M3 values, where only the
    exactly rounded quotient fl32(x / s) decides the code.  The tiles of the
    act_quant brute force (every bf16 magnitude under a fixed maximum) are
    added as well.
    """
    pos = TABLE[:0x7F].astype(np.float64)
    mids = (pos[:-1] + pos[1:]) / 2
    out = []
    rng = np.random.default_rng(41)
    for amax in (np.float32(1.0), np.float32(0.0123), np.float32(3.0e-4), np.float32(17.5)):
        s0 = np.float32(amax / np.float32(448))
        vals = (mids * np.float64(s0)).astype(np.float32)
        vals = np.concatenate([vals, -vals, np.nextafter(vals, np.float32(0)), np.nextafter(vals, np.float32(1e9))])
        vals = vals[np.abs(vals) <= amax]
        vals = rng.permutation(vals)
        n = 128 * (-(-(vals.size + 1) // 128))
        t = np.zeros(n, np.float32)
        t[0] = amax
        t[1:vals.size + 1] = vals
        out.append(t.reshape(-1, 128))
    tb = tiny_blocks()
    for a in np.unique(tb[:, 0]):
        out.append(tb[tb[:, 0] == a][:128])
    return out


def check_exact_quotients(weight_quant, scale_fmt, sample_every: int = 1):
    for x in adversarial_tiles():
        q, s = weight_quant(x, 128, scale_fmt)
        assert s.shape == (1, 1)
        sr = Fraction(float(s[0, 0]))
        amax = max(Fraction(float(np.max(np.abs(x)))), Fraction(float(np.float32(CLAMP))))
        if scale_fmt is None:
            assert s[0, 0] == f32_round(amax / Fraction(DIV))
        else:
            assert sr >= amax / Fraction(DIV) > sr / 2 and np.frexp(float(s[0, 0]))[0] == 0.5
        flat_x, flat_q = x.reshape(-1), q.reshape(-1)
        for i in range(0, flat_x.size, sample_every):
            t = f32_round(Fraction(float(flat_x[i])) / sr)
            assert int(flat_q[i]) == nearest_e4m3_bruteforce(t, TABLE), (float(flat_x[i]), float(t))


@pytest.mark.parametrize("scale_fmt", [None, "ue8m0"])
def test_exact_quotients(scale_fmt):
    check_exact_quotients(oracle.weight_quant, scale_fmt, sample_every=2)


# ---------------------------------------------------------------- round trip

def check_round_trip(weight_quant, scale_fmt):
    x = small_weights(300, 520, seed=22)
    q, s = weight_quant(x, 128, scale_fmt)
    y = oracle.weight_dequant(q, s, 128, out="f32").astype(np.float64)
    srep = np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)[:300, :520]
    t = (x / np.repeat(np.repeat(s, 128, 0), 128, 1)[:300, :520]).astype(np.float32)   # fp32 quotient
    half_ulp = oracle.e4m3.ulp(t.astype(np.float64)) / 2
    fp32_err = np.maximum(np.abs(t.astype(np.float64)) * 2.0**-24, 2.0**-150)
    # + the fp32 rounding of weight_dequant's own product DEC(q) * s
    bound = (half_ulp + fp32_err) * srep + np.abs(y) * 2.0**-24
    assert np.all(np.abs(y - x.astype(np.float64)) <= bound * (1 + 2.0**-40))
    assert np.all(np.abs(t) <= 448.0 * (1 + 2.0**-23))


@pytest.mark.parametrize("scale_fmt", [None, "ue8m0"])
def test_round_trip(scale_fmt):
    check_round_trip(oracle.weight_quant, scale_fmt)


# ---------------------------------------------------------------- torch composition

def torch_weight_quant(x: np.ndarray, scale_fmt):
    m, n = x.shape
    gm, gn = -(-m // 128), -(-n // 128)
    t = torch.zeros(gm * 128, gn * 128, dtype=torch.float32)
    t[:m, :n] = torch.from_numpy(x)
    t4 = t.view(gm, 128, gn, 128)
    amax = t4.abs().amax(dim=(1, 3)).clamp_min(CLAMP)
    s = amax / DIV
    if scale_fmt == "ue8m0":
        mant, e = torch.frexp(s)
        e = torch.where(mant == 0.5, e - 1, e)
        s = torch.ldexp(torch.ones_like(s), e)
    q = (t4 / s[:, None, :, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.reshape(gm * 128, gn * 128)[:m, :n].contiguous().numpy(), s.numpy()


def check_vs_torch(weight_quant, x, scale_fmt):
    q, s = weight_quant(x, 128, scale_fmt)
    tq, ts = torch_weight_quant(x, scale_fmt)
    assert np.array_equal(s.view(np.uint32), ts.view(np.uint32))
    assert np.array_equal(q, tq)


@pytest.mark.parametrize("scale_fmt", [None, "ue8m0"])
def test_vs_torch_composition(scale_fmt):
    check_vs_torch(oracle.weight_quant, small_weights(), scale_fmt)
    check_vs_torch(oracle.weight_quant, small_weights(130, 200, seed=23), scale_fmt)
    check_vs_torch(oracle.weight_quant, gen.weight_quant_workload(1024, 896, dtype="f32")["w"].numpy(), scale_fmt)
