"""GPU parity for fp8_block_gemm_split (split-K for a last round of tiles).

When the 256 x 256 output tiles leave a last round that fills at most half
the compute units, those tiles are computed in 2-4 parts over K and their
FP32 partials added in part order.  Only the summation order differs from
fp8_block_gemm, so every case is held to the oracle bound on rows sampled
inside the split tiles (the tile order is reproduced here to find them), and
ue8m0 against generic scales stays bit-identical.  Cases: 2, 3 and 4 parts,
with and without full rounds, ragged M and N, fp32 and bf16 output, K/128
not a multiple of 4 (per-block scale gathers), a workspace reused dirty, and
the unsplit fallbacks (no workspace, too small a workspace).
"""

import ctypes

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as fb
import oracle
from fp8_block_scaled_quant_amd import _lib
from inputs import gen
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _tile_coords(wg, tiles_m, tiles_n):
    """The tiled kernel's tile order: XCD-aware remap, then 4-row grouped raster."""
    ntiles = tiles_m * tiles_n
    tile = (wg % 8) * (ntiles // 8) + wg // 8 if ntiles % 8 == 0 else wg
    group = tile // (4 * tiles_n)
    first_m = group * 4
    gm = min(tiles_m - first_m, 4)
    idx = tile - group * 4 * tiles_n
    return first_m + idx % gm, idx // gm


def _tail_rows(m, n, count, seed):
    """Rows inside the tiles of the last (split) round."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles_m, tiles_n = -(-m // 256), -(-n // 256)
    ntiles = tiles_m * tiles_n
    full = ntiles // cus * cus
    bands = sorted({_tile_coords(w, tiles_m, tiles_n)[0] for w in range(full, ntiles)})
    rng = np.random.default_rng(seed)
    rows = []
    for tm in bands:
        lo, hi = 256 * tm, min(256 * tm + 256, m)
        rows += [lo, hi - 1] + list(rng.integers(lo, hi, size=max(1, count // len(bands))))
    return np.unique(np.array(rows))


def _check(got, an, asn, w, ws, rows, out):
    c = oracle.fp8_gemm(an, asn, w, ws, rows=rows)
    tol = oracle.gemm_tolerance(an, asn, w, ws, rows=rows)
    ok = oracle.gemm_check(got[rows], c, tol, out)
    assert ok.all(), f"{int((~ok).sum())} sampled outputs out of the bound"


# (m, n, k, out, scale_fmt): 272 tiles = 256 + a tail of 16 (on 256 CUs) in
# 4 parts (K = 8192), 3 parts (K = 6144; ragged and K/128 = 50, no scale
# table, K = 6400); 8 tiles and no full round (K = 8192, 4 parts); a tail of
# 5 (261 tiles: not whole XCD shares, the plain tile-by-part mapping); K/128 =
# 45, two uneven parts (24 and 21 K blocks) without the scale table
@pytest.mark.parametrize("m,n,k,out,scale_fmt", [
    (4096, 4352, 8192, "bf16", "ue8m0"),
    (4096, 4352, 6144, "f32", None),
    (4000, 4300, 6400, "bf16", None),
    (512, 1024, 8192, "f32", "ue8m0"),
    (2304, 7424, 4096, "bf16", "ue8m0"),
    (4096, 4352, 5760, "bf16", "ue8m0"),
])
def test_split_matches_oracle(m, n, k, out, scale_fmt):
    d = gen.custom_gemm(seed=m + n + k, m=m, n=n, k=k, outliers=True)
    G.announce(f"gemm_split m={m} n={n} k={k} out={out} scale_fmt={scale_fmt}")
    dev = G.device()
    a, a_s = fb.act_quant(d["x"].to(dev), 128, scale_fmt)
    a = a.view(torch.uint8)
    assert _lib.lib().fp8_block_gemm_split_workspace(m, n, k) > 0, "shape expected to split"
    got, _ = G.block_gemm_split(a, a_s, d["w"], d["w_s"], out, ue8m0=scale_fmt == "ue8m0")
    an, asn = a.cpu().numpy(), a_s.cpu().numpy()
    _check(got, an, asn, d["w"], d["w_s"], _tail_rows(m, n, 24, m), out)
    if scale_fmt == "ue8m0":
        generic, _ = G.block_gemm_split(a, a_s, d["w"], d["w_s"], out, ue8m0=False)
        assert np.array_equal(got.view(np.uint64), generic.view(np.uint64))


def test_workspace_reused_dirty_and_fallbacks():
    m, n, k = 4096, 4352, 8192
    dev = G.device()
    G.announce("gemm_split workspace reuse and fallbacks")
    d1 = gen.custom_gemm(seed=1, m=m, n=n, k=k)
    x2 = gen.activations(np.random.default_rng(2), m, k)
    a1, s1 = fb.act_quant(d1["x"].to(dev), 128, "ue8m0")
    a2, s2 = fb.act_quant(x2.to(dev), 128, "ue8m0")
    a1, a2 = a1.view(torch.uint8), a2.view(torch.uint8)
    # the guarded workspace starts full of canary bytes: nothing is zeroed for the call
    got1, ws = G.block_gemm_split(a1, s1, d1["w"], d1["w_s"], "bf16", ue8m0=True)
    got2, _ = G.block_gemm_split(a2, s2, d1["w"], d1["w_s"], "bf16", ue8m0=True, ws=ws)
    rows = _tail_rows(m, n, 16, 3)
    _check(got1, a1.cpu().numpy(), s1.cpu().numpy(), d1["w"], d1["w_s"], rows, "bf16")
    _check(got2, a2.cpu().numpy(), s2.cpu().numpy(), d1["w"], d1["w_s"], rows, "bf16")
    # too small a workspace, or none: the unsplit launch, bit for bit
    unsplit = G.block_gemm(None, None, d1["w"], d1["w_s"], "bf16", a_dev=a1, a_s_dev=s1, ue8m0=True)
    need = _lib.lib().fp8_block_gemm_split_workspace(m, n, k)
    small, _ = G.block_gemm_split(a1, s1, d1["w"], d1["w_s"], "bf16", ue8m0=True, ws_bytes=need - 256)
    assert np.array_equal(small.view(np.uint64), unsplit.view(np.uint64))
    c = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    w, wsc = torch.from_numpy(d1["w"]).to(dev), torch.from_numpy(d1["w_s"]).to(dev)
    st = _lib.lib().fp8_block_gemm_split(
        ctypes.c_void_p(a1.data_ptr()), ctypes.c_void_p(s1.data_ptr()), ctypes.c_void_p(w.data_ptr()),
        ctypes.c_void_p(wsc.data_ptr()), ctypes.c_void_p(c.data_ptr()), _lib.BF16, m, n, k, _lib.SCALE_UE8M0,
        None, 0, G.stream())
    assert st == _lib.OK
    torch.cuda.synchronize()
    none = c.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(none.view(np.uint64), unsplit.view(np.uint64))


def test_prefill_shape2_through_binding():
    """8192 x 7168 x 18432: 896 tiles, 768 in full rounds and 128 split in two."""
    d = gen.prefill_gemm(2)
    G.announce("fp8_gemm binding prefill shape 2 (split tail)")
    dev = G.device()
    m, k = d["x"].shape
    n = d["w"].shape[0]
    assert _lib.lib().fp8_block_gemm_split_workspace(m, n, k) > 0
    a, a_s = fb.act_quant(d["x"].to(dev), 128, "ue8m0")
    w, ws = torch.from_numpy(d["w"]).to(dev), torch.from_numpy(d["w_s"]).to(dev)
    c = fb.fp8_gemm(a, a_s, w, ws, torch.bfloat16, "ue8m0")
    c_unsplit = fb.fp8_gemm(a, a_s, w, ws, torch.bfloat16, "ue8m0", split=False)
    got = c.float().cpu().numpy().astype(np.float64)
    an, asn = a.view(torch.uint8).cpu().numpy(), a_s.cpu().numpy()
    _check(got, an, asn, d["w"], d["w_s"], _tail_rows(m, n, 32, 5), "bf16")
    # outside the split tiles the two calls run the same kernel
    tiles_m, tiles_n = -(-m // 256), -(-n // 256)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    full = tiles_m * tiles_n // cus * cus
    tm, tn = _tile_coords(0, tiles_m, tiles_n)
    assert 0 < full
    blk = (slice(256 * tm, 256 * tm + 256), slice(256 * tn, 256 * tn + 256))
    assert torch.equal(c[blk], c_unsplit[blk])
