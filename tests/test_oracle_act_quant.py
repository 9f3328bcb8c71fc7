"""Pins for the oracle's act_quant.

* closed forms the pages fix: an all-zero block gets s = fl32(fl32(1e-4)/448)
  (computed here in exact rational arithmetic), ue8m0 gives 2^-22; a block's
  largest element lands on +-448 exactly (scale_fmt None) or within [224, 448]
  (ue8m0); scales have one value per 1x128 block (page example shape [1,1024]);
* invariants brute-forced on tiny inputs: every bf16 magnitude placed in
  blocks with fixed maxima; each code is the E4M3 value nearest to the fp32
  quotient (brute-force search over torch's table); that quotient is the exact
  x/s rounded once to fp32; ue8m0 scales are powers of two with
  s >= amax/448 > s/2; quantize -> dequantize error <= half an E4M3 ulp x s;
* a second, independent CPU composition of the same definition through torch's
  own ops (amax, clamp, division, frexp, fp8 cast) gives bit-identical output.
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

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
with open(os.path.join(GOLDEN, "page_facts.json")) as _f:
    FACTS = json.load(_f)

CLAMP = FACTS["amax_clamp_min"]["value"]
DIV = FACTS["scale_formula"]["divisor"]
TABLE = torch_e4m3_table()


def _bits(v) -> int:
    return int(np.float32(v).view(np.uint32))


# ---------------------------------------------------------------- closed forms

def zero_block_scale_exact() -> np.float32:
    """fl32(fl32(1e-4) / 448) by exact rational arithmetic."""
    return f32_round(Fraction(float(np.float32(CLAMP))) / Fraction(DIV))


def check_zero_block(act_quant):
    x = np.zeros((2, 256), dtype=np.float32)
    x[1, 128:] = 1.0
    q, s = act_quant(x, 128, None)
    assert _bits(s[0, 0]) == _bits(zero_block_scale_exact()) == 0x346FACAD
    assert np.all(q[0] == 0)
    qu, su = act_quant(x, 128, "ue8m0")
    assert _bits(su[0, 0]) == 0x34800000          # 2^-22: smallest power of two >= 2.23e-7
    assert np.all(qu[0] == 0)
    # a negative zero keeps its sign
    x2 = np.zeros((1, 128), dtype=np.float32)
    x2[0, 5] = -0.0
    q2, _ = act_quant(x2, 128, None)
    assert q2[0, 5] == 0x80 and q2[0, 4] == 0x00


def check_block_max_hits_448(act_quant):
    rng = np.random.default_rng(11)
    x = gen.to_bf16(rng.standard_normal((64, 1024), dtype=np.float32) * 3).float().numpy()
    x[5, :128] *= 1e-6                       # a block below the clamp
    q, s = act_quant(x, 128, None)
    qb = q.reshape(64, 8, 128)
    xb = np.abs(x.reshape(64, 8, 128))
    idx = np.argmax(xb, axis=-1)
    top = np.take_along_axis(qb, idx[..., None], -1)[..., 0]
    amax = xb.max(-1)
    big = amax >= np.float32(CLAMP)
    assert np.all((top[big] & 0x7F) == 0x7E)
    assert not np.all((top[~big] & 0x7F) == 0x7E)
    qu, su = act_quant(x, 128, "ue8m0")
    topu = np.take_along_axis(qu.reshape(64, 8, 128), idx[..., None], -1)[..., 0] & 0x7F
    assert np.all((topu[big] >= 0x76) & (topu[big] <= 0x7E))
    assert s.shape == su.shape == (64, 8)


def check_page_example_shape(act_quant):
    ex = FACTS["act_quant_example"]
    x = np.random.default_rng(0).standard_normal(ex["x_shape"], dtype=np.float32)
    q, s = act_quant(x, ex["block_size"], None)
    assert q.shape == tuple(ex["x_shape"]) and q.dtype == np.uint8
    assert s.shape == (1, ex["scales_per_row_derived"]) and s.dtype == np.float32
    # N-D input: scales keep the leading shape
    x3 = np.random.default_rng(1).standard_normal((2, 3, 256), dtype=np.float32)
    q3, s3 = act_quant(x3, 128, None)
    q2, s2 = act_quant(x3.reshape(6, 256), 128, None)
    assert s3.shape == (2, 3, 2) and np.array_equal(q3.reshape(6, 256), q2)
    assert np.array_equal(s3.reshape(6, 2), s2)


def test_zero_block():
    check_zero_block(oracle.act_quant)


def test_block_max_hits_448():
    check_block_max_hits_448(oracle.act_quant)


def test_page_example_shape():
    check_page_example_shape(oracle.act_quant)


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.act_quant(np.zeros((1, 100), np.float32))
    with pytest.raises(ValueError):
        oracle.act_quant(np.full((1, 128), np.nan, np.float32))
    with pytest.raises(ValueError):
        oracle.act_quant(np.zeros((1, 128), np.float32), scale_fmt="e5m2")


# ---------------------------------------------------------------- brute force

def tiny_blocks() -> np.ndarray:
    """Every finite bf16 value, spread over blocks whose maxima are fixed."""
    bits = np.arange(65536, dtype=np.uint32) << 16
    allv = bits.view(np.float32)
    allv = allv[np.isfinite(allv)]
    rows = []
    for amax in (np.float32(1.0), np.float32(3.1875), np.float32(448.0 * 0.75),
                 np.float32(2.0**-20), np.float32(7.0e-5), np.float32(1e4)):
        vals = allv[np.abs(allv) <= amax]
        rng = np.random.default_rng(int(amax * 1000) % 2**31)
        vals = rng.choice(vals, size=min(vals.size, 127 * 24), replace=False)
        nblk = -(-vals.size // 127)
        pad = np.zeros(nblk * 127, np.float32)
        pad[:vals.size] = vals
        blk = np.concatenate([np.full((nblk, 1), amax, np.float32), pad.reshape(nblk, 127)], axis=1)
        rows.append(blk)
    return np.concatenate(rows, 0)          # [n, 128]


def check_invariants(act_quant, scale_fmt, sample_every: int = 1):
    x = tiny_blocks()
    q, s = act_quant(x, 128, scale_fmt)
    s = s[:, 0]
    for r in range(x.shape[0]):
        amax = Fraction(float(max(np.max(np.abs(x[r])), np.float32(CLAMP))))
        sr = Fraction(float(s[r]))
        if scale_fmt is None:
            assert s[r] == f32_round(amax / Fraction(DIV))
        else:
            m, _ = np.frexp(float(s[r]))
            assert m == 0.5                                 # power of two
            assert sr >= amax / Fraction(DIV) > sr / 2
        for c in range(0, 128, sample_every):
            exact = Fraction(float(x[r, c])) / sr
            t = f32_round(exact)
            # fp32 quotient: exact quotient rounded once (half an ulp; fp32 subnormals are absolute)
            rnd = max(abs(exact) * Fraction(1, 2**24), Fraction(1, 2**150))
            assert abs(Fraction(float(t)) - exact) <= rnd
            code = int(q[r, c])
            assert code == nearest_e4m3_bruteforce(t, TABLE), (r, c, x[r, c], float(t))
            # quantize -> dequantize error: half an E4M3 ulp of the quotient plus the fp32 rounding
            deq = Fraction(float(TABLE[code])) * sr
            xv = Fraction(float(x[r, c]))
            half_ulp = Fraction(float(oracle.e4m3.ulp(np.array([float(t)]))[0])) / 2
            assert abs(deq - xv) <= (half_ulp + rnd) * sr


@pytest.mark.parametrize("scale_fmt", [None, "ue8m0"])
def test_invariants_bruteforce(scale_fmt):
    check_invariants(oracle.act_quant, scale_fmt, sample_every=3)


# ---------------------------------------------------------------- torch composition

def torch_act_quant(x: np.ndarray, scale_fmt):
    t = torch.from_numpy(x).reshape(-1, x.shape[-1] // 128, 128)
    amax = t.abs().amax(-1).clamp_min(CLAMP)
    s = amax / DIV
    if scale_fmt == "ue8m0":
        m, e = torch.frexp(s)
        e = torch.where(m == 0.5, e - 1, e)
        s = torch.ldexp(torch.ones_like(s), e)
    q = (t / s[..., None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.reshape(x.shape).numpy(), s.reshape(x.shape[:-1] + (x.shape[-1] // 128,)).numpy()


def check_vs_torch(act_quant, x, scale_fmt):
    q, s = act_quant(x, 128, scale_fmt)
    tq, ts = torch_act_quant(x, scale_fmt)
    assert np.array_equal(s.view(np.uint32), ts.view(np.uint32))
    assert np.array_equal(q, tq)


@pytest.mark.parametrize("scale_fmt", [None, "ue8m0"])
def test_vs_torch_composition(scale_fmt):
    x = gen.act_quant_workload(m=512, k=7168, seed=99)["x"].float().numpy()
    check_vs_torch(oracle.act_quant, x, scale_fmt)
    check_vs_torch(oracle.act_quant, tiny_blocks(), scale_fmt)
    tiny = gen.tiny_gemm()["x"].numpy()
    check_vs_torch(oracle.act_quant, tiny, scale_fmt)
