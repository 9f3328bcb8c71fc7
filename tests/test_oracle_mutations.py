"""Planted mistakes: each plausible slip in the oracle must fail some pin.

Every case below plants one mistake in the oracle (on the CPU, through
monkeypatching or a one-line variant of an oracle function) and asserts that at
least one of the pin checks from the other oracle test modules rejects it.
"""

import numpy as np
import pytest

import importlib

import oracle
from oracle import e4m3

aq_mod = importlib.import_module("oracle.act_quant")
dq_mod = importlib.import_module("oracle.weight_dequant")
from inputs import gen
from tests import test_oracle_act_quant as T_aq
from tests import test_oracle_dequant as T_dq
from tests import test_oracle_e4m3 as T_e4
from tests import test_oracle_gemm as T_g


def _fails(fn, *args):
    try:
        fn(*args)
    except (AssertionError, ValueError):
        return True
    return False


def _any_act_quant_pin_fails(act_quant):
    x = gen.act_quant_workload(m=256, k=1024, seed=5)["x"].float().numpy()
    checks = [
        (T_aq.check_zero_block, (act_quant,)),
        (T_aq.check_block_max_hits_448, (act_quant,)),
        (T_aq.check_invariants, (act_quant, None, 5)),
        (T_aq.check_invariants, (act_quant, "ue8m0", 5)),
        (T_aq.check_vs_torch, (act_quant, x, None)),
        (T_aq.check_vs_torch, (act_quant, x, "ue8m0")),
    ]
    return any(_fails(f, *a) for f, a in checks)


# --------------------------------------------------------------- encoder

def _encode_ties_away(v):
    v = np.asarray(v)
    a = np.abs(v.astype(np.float64))
    idx = np.clip(np.searchsorted(e4m3._POS, a, side="right") - 1, 0, 0x7E)
    nxt = np.minimum(idx + 1, 0x7E)
    mid = (e4m3._POS[idx] + e4m3._POS[nxt]) / 2
    code = np.where(a >= mid, nxt, idx)
    code = np.where(a >= 448, 0x7E, code) | (np.signbit(v).astype(np.int64) << 7)
    return code.astype(np.uint8)


def _encode_no_signed_zero(v):
    c = _REAL_ENCODE(v)
    return np.where((c & 0x7F) == 0, 0, c).astype(np.uint8)


def _encode_nan_overflow(v):
    c = _REAL_ENCODE(v)
    return np.where(np.abs(np.asarray(v, np.float64)) > 448, 0x7F, c).astype(np.uint8)


_REAL_ENCODE = e4m3.encode


@pytest.mark.parametrize("mutant", [_encode_ties_away, _encode_no_signed_zero, _encode_nan_overflow])
def test_encoder_mutants_caught(mutant):
    checks = [
        (T_e4.check_encode_round_trip, (mutant,)),
        (T_e4.check_encode_vs_torch, (mutant, T_e4.all_bf16_as_f32())),
        (T_e4.check_encode_vs_torch, (mutant, T_e4.midpoint_sweep(8))),
    ]
    caught = any(_fails(f, *a) for f, a in checks)
    if not caught:   # the tie / zero / saturation table
        def table_check():
            for v, code in [(1.0625, 0x38), (-0.0, 0x80), (460.0, 0x7E), (1e30, 0x7E)]:
                assert int(mutant(np.array([v], np.float32))[0]) == code
        caught = _fails(table_check)
    assert caught


def test_table_mutant_caught():
    bad = e4m3.DECODE.copy()
    bad[0x01] = 2.0**-10          # subnormal step off by one exponent
    assert _fails(T_e4.check_table, bad)
    bad = e4m3.DECODE.copy()
    bad[0x7E] = 480.0             # the FN top code treated as IEEE-like
    assert _fails(T_e4.check_table, bad)


# --------------------------------------------------------------- act_quant

def test_clamp_constant_mutant(monkeypatch):
    monkeypatch.setattr(aq_mod, "_CLAMP", np.float32(1e-5))
    assert _any_act_quant_pin_fails(oracle.act_quant)


def test_max_constant_mutant(monkeypatch):
    monkeypatch.setattr(aq_mod, "_FP8_MAX", np.float32(480.0))
    assert _any_act_quant_pin_fails(oracle.act_quant)


def test_ue8m0_round_down_mutant(monkeypatch):
    def floor_pow2(s):
        m, e = np.frexp(s.astype(np.float64))
        return np.ldexp(1.0, e - 1).astype(np.float32)
    monkeypatch.setattr(aq_mod, "_ue8m0_round_up", floor_pow2)
    assert _any_act_quant_pin_fails(oracle.act_quant)


def test_ue8m0_nearest_mutant(monkeypatch):
    def nearest_pow2(s):
        return (2.0 ** np.round(np.log2(s.astype(np.float64)))).astype(np.float32)
    monkeypatch.setattr(aq_mod, "_ue8m0_round_up", nearest_pow2)
    assert _any_act_quant_pin_fails(oracle.act_quant)


def test_encoder_ties_away_inside_act_quant(monkeypatch):
    monkeypatch.setattr(e4m3, "encode", _encode_ties_away)
    assert _any_act_quant_pin_fails(oracle.act_quant)


def _act_quant_reciprocal(x, block_size=128, scale_fmt=None):
    """Variant: multiplies by fl32(1/s) instead of dividing by s."""
    nb = x.shape[-1] // block_size
    xb = x.reshape(-1, nb, block_size)
    amax = np.maximum(np.max(np.abs(xb), -1), np.float32(1e-4))
    s = (amax / np.float32(448)).astype(np.float32)
    if scale_fmt == "ue8m0":
        s = aq_mod._ue8m0_round_up(s)
    inv = (np.float32(1) / s).astype(np.float32)
    q = e4m3.encode((xb * inv[:, :, None]).astype(np.float32))
    return q.reshape(x.shape), s.reshape(x.shape[:-1] + (nb,))


def _act_quant_clamp_after(x, block_size=128, scale_fmt=None):
    """Variant: clamps the scale instead of amax."""
    nb = x.shape[-1] // block_size
    xb = x.reshape(-1, nb, block_size)
    s = np.maximum((np.max(np.abs(xb), -1) / np.float32(448)).astype(np.float32), np.float32(1e-4))
    if scale_fmt == "ue8m0":
        s = aq_mod._ue8m0_round_up(s)
    q = e4m3.encode((xb / s[:, :, None]).astype(np.float32))
    return q.reshape(x.shape), s.reshape(x.shape[:-1] + (nb,))


@pytest.mark.parametrize("mutant", [_act_quant_reciprocal, _act_quant_clamp_after])
def test_act_quant_variants_caught(mutant):
    assert _any_act_quant_pin_fails(mutant)


# --------------------------------------------------------------- weight_dequant

def _dequant_any_fails(weight_dequant):
    checks = [
        (T_dq.check_page_grid, (weight_dequant,)),
        (T_dq.check_ragged_grid, (weight_dequant,)),
        (T_dq.check_unit_and_pow2, (weight_dequant,)),
        (T_dq.check_tile_mapping, (weight_dequant,)),
        (T_dq.check_vs_torch, (weight_dequant, 300, 520, 12)),
    ]
    return any(_fails(f, *a) for f, a in checks)


def test_dequant_divides_mutant():
    def mutant(x, s, block_size=128, out="f32"):
        return oracle.weight_dequant(x, (np.float32(1) / s).astype(np.float32), block_size, out)
    assert _dequant_any_fails(mutant)


def test_dequant_transposed_grid_mutant():
    def mutant(x, s, block_size=128, out="f32"):
        m, n = x.shape
        y = oracle.weight_dequant(x, np.ones_like(s), block_size, "f32")
        gm, gn = s.shape
        flat = s.reshape(-1)
        col_major = np.array([[flat[(j * gm + i) % flat.size] for j in range(gn)] for i in range(gm)], np.float32)
        full = np.repeat(np.repeat(col_major, block_size, 0)[:m], block_size, 1)[:, :n]
        y = (y * full).astype(np.float32)
        return dq_mod.f32_to_bf16_bits(y) if out == "bf16" else y
    assert _dequant_any_fails(mutant)


def test_dequant_truncating_bf16_mutant(monkeypatch):
    monkeypatch.setattr(dq_mod, "f32_to_bf16_bits",
                        lambda v: (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16))
    assert _dequant_any_fails(oracle.weight_dequant)


# --------------------------------------------------------------- GEMM

def _gemm_any_fails(fp8_gemm):
    checks = [
        (T_g.check_exact, (fp8_gemm, 2, 4, 4, 384)),
        (T_g.check_vs_dequant_matmul, (fp8_gemm, 11, 33, 300, 1024)),
        (T_g.check_single_block, (fp8_gemm,)),
        (T_g.check_integer_codes, (fp8_gemm,)),
        (T_g.check_homogeneity, (fp8_gemm,)),
    ]
    return any(_fails(f, *a) for f, a in checks)


def test_gemm_drops_activation_scale():
    def mutant(a, a_s, b, b_s, block_size=128, rows=None):
        return oracle.fp8_gemm(a, np.ones_like(a_s), b, b_s, block_size, rows)
    assert _gemm_any_fails(mutant)


def test_gemm_wrong_weight_scale_block():
    def mutant(a, a_s, b, b_s, block_size=128, rows=None):
        # uses the first weight block-row's scales for every column
        return oracle.fp8_gemm(a, a_s, b, np.repeat(b_s[:1], b_s.shape[0], 0), block_size, rows)
    assert _gemm_any_fails(mutant)


def test_gemm_shifted_k_block_scale(monkeypatch):
    def mutant(a, a_s, b, b_s, block_size=128, rows=None):
        return oracle.fp8_gemm(a, np.roll(a_s, 1, axis=1), b, b_s, block_size, rows)
    assert _gemm_any_fails(mutant)


def test_gemm_reversed_k_in_one_operand():
    def mutant(a, a_s, b, b_s, block_size=128, rows=None):
        return oracle.fp8_gemm(a, a_s, np.ascontiguousarray(b[:, ::-1]), b_s, block_size, rows)
    assert _gemm_any_fails(mutant)


def test_gemm_decode_sign_lost(monkeypatch):
    monkeypatch.setattr(e4m3, "decode", lambda c: np.abs(e4m3.DECODE[np.asarray(c)]))
    assert _gemm_any_fails(oracle.fp8_gemm)


# --------------------------------------------------------------- weight quant

from tests import test_oracle_weight_quant as T_wq  # noqa: E402


def _wq_any_fails(weight_quant):
    checks = [
        (T_wq.check_identical_rows_match_act_quant, (weight_quant, None)),
        (T_wq.check_identical_rows_match_act_quant, (weight_quant, "ue8m0")),
        (T_wq.check_zero_tile, (weight_quant,)),
        (T_wq.check_tile_max_hits_448, (weight_quant,)),
        (T_wq.check_grid_and_edge_tiles, (weight_quant,)),
        (T_wq.check_round_trip, (weight_quant, None)),
        (T_wq.check_round_trip, (weight_quant, "ue8m0")),
        (T_wq.check_vs_torch, (weight_quant, T_wq.small_weights(), None)),
        (T_wq.check_vs_torch, (weight_quant, T_wq.small_weights(), "ue8m0")),
        (T_wq.check_exact_quotients, (weight_quant, None, 3)),
        (T_wq.check_exact_quotients, (weight_quant, "ue8m0", 3)),
    ]
    return any(_fails(f, *a) for f, a in checks)


def _wq_variant(amax_of=None, quotient=None, clamp_after_div=False, ue8m0_down=False, tiles_of=None):
    """The oracle's weight_quant with one step replaced."""
    def wq(x, block_size=128, scale_fmt=None):
        m, n = x.shape
        bs = block_size
        gm, gn = -(-m // bs), -(-n // bs)
        xp = np.zeros((gm * bs, gn * bs), dtype=np.float32)
        xp[:m, :n] = x
        tiles = tiles_of(xp, gm, gn, bs) if tiles_of else xp.reshape(gm, bs, gn, bs)
        amax = amax_of(tiles) if amax_of else np.max(np.abs(tiles), axis=(1, 3))
        if clamp_after_div:
            s = np.maximum((amax / np.float32(448)).astype(np.float32), np.float32(1e-4))
        else:
            s = (np.maximum(amax, np.float32(1e-4)) / np.float32(448)).astype(np.float32)
        if scale_fmt == "ue8m0":
            if ue8m0_down:
                s = np.ldexp(np.float32(1.0), np.frexp(s.astype(np.float64))[1] - 1).astype(np.float32)
            else:
                s = wq_mod._ue8m0_round_up(s)
        sb = s[:, None, :, None]
        q = quotient(tiles, sb) if quotient else (tiles / sb).astype(np.float32)
        if tiles_of:   # back to the padded matrix's element order
            q = q.transpose(0, 2, 1, 3)
        codes = e4m3.encode(q).reshape(gm * bs, gn * bs)[:m, :n]
        return np.ascontiguousarray(codes), s
    return wq


wq_mod = importlib.import_module("oracle.weight_quant")


def test_wq_variant_harness_is_faithful():
    """With nothing replaced, the variant builder reproduces the oracle."""
    x = T_wq.small_weights(300, 520, seed=31)
    for fmt in (None, "ue8m0"):
        q, s = _wq_variant()(x, 128, fmt)
        q0, s0 = oracle.weight_quant(x, 128, fmt)
        assert np.array_equal(q, q0) and np.array_equal(s, s0)


@pytest.mark.parametrize("name, mutant", [
    ("amax of the tile's first row only", _wq_variant(amax_of=lambda t: np.max(np.abs(t[:, :1]), axis=(1, 3)))),
    ("signed max instead of magnitude", _wq_variant(amax_of=lambda t: np.max(t, axis=(1, 3)))),
    ("clamp applied to the scale", _wq_variant(clamp_after_div=True)),
    ("multiply by fl32(1/s)", _wq_variant(quotient=lambda t, sb: (t * (np.float32(1) / sb).astype(np.float32)).astype(np.float32))),
    ("ue8m0 rounded down", _wq_variant(ue8m0_down=True)),
    # contiguous runs of 16384 elements taken as the tiles (a reshape slip)
    ("16384-element strips instead of 128 x 128 tiles",
     _wq_variant(tiles_of=lambda xp, gm, gn, bs: xp.reshape(gm, gn, bs, bs).transpose(0, 2, 1, 3))),
])
def test_weight_quant_mutants_caught(name, mutant):
    assert _wq_any_fails(mutant), name


# --------------------------------------------------------------- bf16 bound

from tests import test_oracle_bf16 as T_bf  # noqa: E402

gemm_mod = importlib.import_module("oracle.fp8_gemm")


def _bf16_bound_any_fails():
    checks = [
        (T_bf.check_ulp_spacing, (gemm_mod.bf16_ulp,)),
        (T_bf.check_ulp_special, (gemm_mod.bf16_ulp,)),
        (T_bf.check_gemm_bound_bf16, (oracle.gemm_check,)),
        (T_bf.check_ulp_taken_at_c, (oracle.gemm_check,)),
    ]
    return any(_fails(f, *a) for f, a in checks)


def _ulp_with(exp_shift=7, floor=-126, log2=False):
    """bf16_ulp with one step replaced."""
    def ulp(v):
        a = np.abs(np.asarray(v, dtype=np.float64))
        if log2:   # exponent from a rounded log2
            e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
        else:
            e = np.frexp(a)[1].astype(np.int64) - 1
        e = np.maximum(np.where(a > 0, e, floor), floor)
        return np.ldexp(1.0, e - exp_shift)
    return ulp


def test_bf16_ulp_variant_harness_is_faithful():
    v = np.concatenate([np.ldexp(1.0, np.arange(-140, 130)), [0.0, 3.0, -5.5, 1e-45]])
    assert np.array_equal(_ulp_with()(v), gemm_mod.bf16_ulp(v))


@pytest.mark.parametrize("name, mutant", [
    ("two ulps (e - 6)", _ulp_with(exp_shift=6)),
    ("half an ulp (e - 8)", _ulp_with(exp_shift=8)),
    ("exponent from a rounded log2", _ulp_with(log2=True)),
    ("fp32 subnormal floor instead of bf16's", _ulp_with(floor=-149)),
    ("no subnormal floor at the normal boundary", _ulp_with(floor=-127)),
])
def test_bf16_ulp_mutants_caught(name, mutant, monkeypatch):
    monkeypatch.setattr(gemm_mod, "bf16_ulp", mutant)
    assert _bf16_bound_any_fails(), name


def test_gemm_check_ulp_of_gpu_value_caught():
    def mutant(gpu, c, tol, out="f32"):
        gpu = np.asarray(gpu, dtype=np.float64)
        bound = tol + (gemm_mod.bf16_ulp(gpu) if out == "bf16" else 0.0)
        return np.isfinite(gpu) & (np.abs(gpu - c) <= bound)
    assert _fails(T_bf.check_ulp_taken_at_c, mutant)


def test_gemm_check_ignores_ulp_caught():
    def mutant(gpu, c, tol, out="f32"):
        gpu = np.asarray(gpu, dtype=np.float64)
        return np.isfinite(gpu) & (np.abs(gpu - c) <= tol)
    assert _fails(T_bf.check_gemm_bound_bf16, mutant)


@pytest.mark.parametrize("name, mutant", [
    ("sign bit dropped", lambda b: ((np.asarray(b, np.uint16).astype(np.uint32) & 0x7FFF) << 16).view(np.float32)),
    ("shifted by 15", lambda b: (np.asarray(b, np.uint16).astype(np.uint32) << 15).view(np.float32)),
    ("bytes swapped", lambda b: (np.asarray(b, np.uint16).byteswap().astype(np.uint32) << 16).view(np.float32)),
])
def test_bf16_bits_to_f32_mutants_caught(name, mutant):
    assert _fails(T_bf.check_bits_to_f32, mutant), name
