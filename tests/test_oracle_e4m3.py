"""Pins for the oracle's E4M3 table and encoder.

* the table against the format's fixed code points (golden fixture) and the
  pages' 448 maximum, and against torch's CPU float8_e4m3fn decode (a library
  special case of the same format);
* the encoder: round trip over all finite codes, exhaustive over all 65536
  bf16 bit patterns and a dense fp32 sweep around every rounding midpoint
  against torch's CPU cast (which agrees with RNE-with-saturation wherever
  |v| <= 464; above that torch gives NaN and the oracle saturates), and
  brute-force nearest-value search on samples.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import e4m3
from tests.exact import nearest_e4m3_bruteforce, torch_e4m3_table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_value(text: str) -> float:
    if text == "nan":
        return float("nan")
    if text == "-0":
        return -0.0
    neg = text.startswith("-")
    t = text.lstrip("-")
    if "^" in t:
        coef, _, pw = t.partition("2^")
        coef = float(coef.rstrip("*")) if coef else 1.0
        v = coef * 2.0 ** int(pw)
    else:
        v = float(t)
    return -v if neg else v


def check_table(decode_table):
    with open(os.path.join(GOLDEN, "e4m3_format_codes.json")) as f:
        fixture = json.load(f)["codes"]
    for code_hex, text in fixture:
        want = _golden_value(text)
        got = decode_table[int(code_hex, 16)]
        if np.isnan(want):
            assert np.isnan(got), code_hex
        else:
            assert got == want and np.signbit(got) == np.signbit(want), (code_hex, got, want)
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        facts = json.load(f)
    finite = decode_table[np.isfinite(decode_table)]
    assert finite.max() == facts["e4m3_max"]["value"]
    assert finite.min() == -facts["e4m3_max"]["value"]
    assert finite.size == 254 and not np.any(np.isinf(decode_table))
    torch_tab = torch_e4m3_table()
    both_nan = np.isnan(torch_tab) & np.isnan(decode_table)
    assert np.all(both_nan | (torch_tab == decode_table))
    assert np.array_equal(np.signbit(torch_tab[~both_nan]), np.signbit(decode_table[~both_nan]))


def test_decode_table_pinned():
    check_table(e4m3.DECODE)


def _torch_encode(v32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def check_encode_round_trip(encode):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = torch_e4m3_table()[codes].astype(np.float32)
    assert np.array_equal(encode(vals), codes)


def check_encode_vs_torch(encode, v32: np.ndarray):
    v32 = v32[~np.isnan(v32)]
    small = np.abs(v32.astype(np.float64)) <= 464.0
    got = encode(v32)
    assert np.array_equal(got[small], _torch_encode(v32[small]))
    big = ~small
    want_big = np.where(np.signbit(v32[big]), 0xFE, 0x7E).astype(np.uint8)
    assert np.array_equal(got[big], want_big)


def all_bf16_as_f32() -> np.ndarray:
    bits = np.arange(65536, dtype=np.uint32) << 16
    return bits.view(np.float32)


def midpoint_sweep(width: int = 64) -> np.ndarray:
    """Every fp32 within +-width ulps of each midpoint between neighbouring
    positive E4M3 values, of 448 and of 464, with both signs."""
    tab = torch_e4m3_table()[:0x7F]
    mids = (tab[:-1] + tab[1:]) / 2
    centres = np.concatenate([mids, [448.0, 464.0], tab]).astype(np.float32)
    offs = np.arange(-width, width + 1, dtype=np.int64)
    bits = centres.view(np.uint32).astype(np.int64)[:, None] + offs[None, :]
    bits = bits[(bits >= 0)]
    v = bits.astype(np.uint32).view(np.float32)
    return np.concatenate([v, -v])


def test_encode_round_trip():
    check_encode_round_trip(e4m3.encode)


def test_encode_exhaustive_bf16():
    check_encode_vs_torch(e4m3.encode, all_bf16_as_f32())


def test_encode_midpoint_sweep():
    check_encode_vs_torch(e4m3.encode, midpoint_sweep())


def test_encode_random_fp32():
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 2**32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    check_encode_vs_torch(e4m3.encode, bits.view(np.float32))


def test_encode_ties_zero_and_saturation():
    cases = [
        (1.0625, 0x38),          # tie between 1 and 1.125 -> even code 0x38
        (1.1875, 0x3A),          # tie between 1.125 and 1.25 -> even code 0x3A
        (1.5 * 2**-9, 0x02),     # subnormal tie -> even
        (2.0**-10, 0x00),        # half the smallest subnormal ties to zero
        (-2.0**-10, 0x80),       # ... and keeps its sign
        (-0.0, 0x80),
        (0.0, 0x00),
        (2.0**-10 * 1.0000001, 0x01),
        (448.0, 0x7E),
        (460.0, 0x7E),
        (1e30, 0x7E),
        (-1e30, 0xFE),
        (float("inf"), 0x7E),
        (float("-inf"), 0xFE),
    ]
    for v, code in cases:
        assert int(e4m3.encode(np.array([v], dtype=np.float32))[0]) == code, v
    assert int(e4m3.encode(np.array([np.nan], dtype=np.float32))[0]) == 0x7F


def test_encode_bruteforce_samples():
    rng = np.random.default_rng(7)
    tab = torch_e4m3_table()
    v = np.concatenate([
        (rng.standard_normal(300) * 50).astype(np.float32),
        (rng.standard_normal(300) * 2**-8).astype(np.float32),
        midpoint_sweep(2)[::7],
    ])
    got = e4m3.encode(v)
    for x, c in zip(v, got):
        assert int(c) == nearest_e4m3_bruteforce(x, tab), x


@pytest.mark.parametrize("v,want", [(448.0, 32.0), (1.0, 0.125), (2.0**-6, 2.0**-9), (2.0**-8, 2.0**-9)])
def test_ulp(v, want):
    assert e4m3.ulp(np.array([v]))[0] == want
