"""Pins of the oracle's per-row outer scales and 16x16 tile scales against
what the pages state about them ("End-to-End 4-Bit Training": 'Block-scaled
backward passes' for the tiles, 'Recipe details' for per-token / per-expert
outer scales), exact rational arithmetic, and reductions to the already
pinned per-tensor 1x16 quantizer.  CPU only."""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

E4M3, UE5M3 = O.FMT_E4M3, O.FMT_UE5M3


def _bf16(x):
    u = np.asarray(x, np.float32).view(np.uint32)
    return (((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16).view(np.float32)


def _tensor(rows, cols, seed, spread=1.5):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)) * np.exp(rng.normal(0, spread, (rows, 1)))
    x[rng.random((rows, cols)) < 0.01] *= 30
    return _bf16(x.astype(np.float32))


# ---------------------------------------------------------------- per-row outer scales
def test_row_amax_is_the_row_maximum():
    x = _tensor(37, 48, 1)
    assert np.array_equal(O.row_amax(x), np.abs(x).max(axis=1))
    x[3, 5] = np.nan
    x[7, 0] = -np.inf
    ra = O.row_amax(x)
    assert np.isnan(ra[3]) and np.isinf(ra[7]) and ra[7] > 0
    assert np.array_equal(np.delete(ra, [3, 7]), np.delete(np.abs(x).max(axis=1), [3, 7]))


@pytest.mark.parametrize("select,rounding", [(O.SELECT_6, O.ROUND_RNE), (O.SELECT_4OVER6, O.ROUND_RNE),
                                             (O.SELECT_6, O.ROUND_SR)])
def test_rowscaled_is_batch_invariant(pages, select, rounding):
    """A row's codes and scale bytes do not depend on any other row: the
    property the per-token recipe relies on ([E2E] Recipe details)."""
    assert "batch" in pages["per_token_outer_scales"]["note"]
    x = _tensor(40, 64, 2)
    ra = O.row_amax(x)
    kw = dict(select=select, rounding=rounding, seed=99)
    c_all, s_all, _ = O.quantize_rowscaled(x, ra, **kw)
    # a slice of the batch, quantized alone at its global row offset
    c_sub, s_sub, _ = O.quantize_rowscaled(x[11:23], ra[11:23], row0=11, **kw)
    assert np.array_equal(c_sub, c_all[11:23]) and np.array_equal(s_sub, s_all[11:23])
    # changing other rows (even their scale) leaves row 5 untouched
    y = x.copy()
    y[6:] *= 1000.0
    c_y, s_y, _ = O.quantize_rowscaled(y, O.row_amax(y), **kw)
    assert np.array_equal(c_y[:6], c_all[:6]) and np.array_equal(s_y[:6], s_all[:6])


def test_rowscaled_reduces_to_per_tensor_when_rows_share_the_amax():
    x = _tensor(24, 64, 3)
    big = float(np.abs(x).max()) * 1.25
    x[:, 17] = big  # every row now has the same maximum
    x = _bf16(x)
    a = float(np.abs(x).max())
    for select in (O.SELECT_6, O.SELECT_4OVER6):
        c_t, s_t, n_t = O.quantize(x, a, select=select)
        c_r, s_r, n_r = O.quantize_rowscaled(x, np.full(24, a, np.float32), select=select)
        assert np.array_equal(c_t, c_r) and np.array_equal(s_t, s_r) and n_t == n_r


def test_rowscaled_block_holding_the_row_max_gets_the_fp8_max():
    """alpha_r = A_r / (6 S_g) maps each row's largest block to the scale S_g
    (448 = 0x7E for E4M3 under max->6), whatever the row's magnitude."""
    x = _tensor(32, 128, 4, spread=4.0)
    ra = O.row_amax(x)
    _, s, _ = O.quantize_rowscaled(x, ra, select=O.SELECT_6, global_max=448.0)
    blk = np.abs(x).reshape(32, 8, 16).max(axis=2).argmax(axis=1)
    assert all(s[r, blk[r]] == 0x7E for r in range(32))


def test_rowscaled_scale_codes_match_exact_rationals():
    """Each block's scale code is the nearest code to a_b / (6 alpha_r) in
    exact arithmetic, except where binary32 rounding lands near a midpoint."""
    x = _tensor(16, 64, 5, spread=3.0)
    ra = O.row_amax(x)
    _, s, _ = O.quantize_rowscaled(x, ra, select=O.SELECT_6, global_max=448.0)
    dec = [Fraction(O.scale_decode(E4M3, c)) for c in range(0x7F)]
    checked = 0
    for r in range(16):
        al = Fraction(float(np.float32(O.alpha(float(ra[r]), 448.0))))
        for b in range(4):
            ab = Fraction(float(np.abs(x[r, b * 16:(b + 1) * 16]).max()))
            t = ab / (6 * al)
            dist = sorted((abs(d - t), c) for c, d in enumerate(dec))
            if dist[1][0] - dist[0][0] < t * Fraction(1, 1 << 20):
                continue  # too close to a midpoint for binary32 to decide like exact arithmetic
            assert s[r, b] == dist[0][1]
            checked += 1
    assert checked > 50


def test_dequantize_rowscaled_is_fp4_times_fp8_times_fp32():
    x = _tensor(12, 32, 6)
    ra = O.row_amax(x)
    c, s, _ = O.quantize_rowscaled(x, ra, select=O.SELECT_4OVER6)
    xh = O.dequantize_rowscaled(c, s, ra, select=O.SELECT_4OVER6)
    nib = O.unpack_codes(c)
    for r in range(12):
        al = float(np.float32(O.alpha(float(ra[r]), 256.0)))
        for col in range(0, 32, 5):
            want = O.e2m1_value(nib[r, col]) * O.scale_decode(E4M3, s[r, col // 16]) * al
            assert xh[r, col] == np.float32(want)


# ---------------------------------------------------------------- 16x16 tile scales
def _nib_t(codes_t, rows):
    return O.unpack_codes(codes_t)  # [cols, rows]


def test_2d_transpose_is_bit_identical(pages):
    """One scale per 16x16 tile makes the column-wise codes exactly the
    transpose of the row-wise ones ([E2E] Block-scaled backward passes)."""
    assert pages["tile_2d"]["transpose_identical"]
    x = _tensor(64, 96, 7)
    c, s, ct, st = O.quantize_2d(x, O.tensor_amax(x))
    assert np.array_equal(O.unpack_codes(ct), O.unpack_codes(c).T)
    # scale bytes: constant over each tile, and the same tile code both ways
    tiles = s.reshape(4, 16, 6)
    assert (tiles == tiles[:, :1, :]).all()
    tiles_t = st.reshape(6, 16, 4)
    assert (tiles_t == tiles_t[:, :1, :]).all()
    assert np.array_equal(tiles[:, 0, :].T, tiles_t[:, 0, :])


def test_2d_tile_scale_is_the_encoded_tile_amax():
    x = _tensor(48, 48, 8, spread=2.0)
    a = float(O.tensor_amax(x))
    c, s, _, _ = O.quantize_2d(x, a, global_max=448.0)
    al = Fraction(float(np.float32(O.alpha(a, 448.0))))
    dec = [Fraction(O.scale_decode(E4M3, k)) for k in range(0x7F)]
    checked = 0
    for tr in range(3):
        for tc in range(3):
            at = Fraction(float(np.abs(x[tr * 16:(tr + 1) * 16, tc * 16:(tc + 1) * 16]).max()))
            t = at / (6 * al)
            dist = sorted((abs(d - t), k) for k, d in enumerate(dec))
            if dist[1][0] - dist[0][0] < t * Fraction(1, 1 << 20):
                continue
            assert s[tr * 16, tc] == dist[0][1]
            checked += 1
    assert checked >= 8


def test_2d_reduces_to_1x16_when_a_tiles_blocks_share_the_amax():
    x = _tensor(32, 64, 9)
    # give every row block of a tile the tile's maximum
    for tr in range(2):
        for tc in range(4):
            t = x[tr * 16:(tr + 1) * 16, tc * 16:(tc + 1) * 16]
            t[:, 3] = np.abs(t).max() * np.where(np.arange(16) % 2 == 0, 1.0, -1.0)
    x = _bf16(x)
    a = float(O.tensor_amax(x))
    c2, s2, _, _ = O.quantize_2d(x, a)
    c1, s1, _ = O.quantize(x, a, select=O.SELECT_6)
    assert np.array_equal(c2, c1) and np.array_equal(s2, s1)


def test_2d_outlier_and_large_row_tiles(pages):
    """The page's tiles: a single large value among 256 sets the tile scale
    and the other 255 values round to zero; a full row of large values keeps
    only that row (under 1x16 row blocks every value survives)."""
    t = pages["tile_2d"]
    rng = np.random.default_rng(0)
    small = rng.uniform(0.5, 1.5, (16, 16)).astype(np.float32)
    tile = small.copy()
    tile[7, 3] = 1000.0
    c, _, _, _ = O.quantize_2d(tile, 1000.0)
    assert int((O.unpack_codes(c) & 7 != 0).sum()) == t["one_outlier_2d_survivors"]
    tile = small.copy()
    tile[5, :] = 1000.0
    c, _, _, _ = O.quantize_2d(tile, 1000.0)
    assert int((O.unpack_codes(c) & 7 != 0).sum()) == t["row_of_large_2d_survivors"]
    c1, _, _ = O.quantize(tile, 1000.0, select=O.SELECT_6)
    assert int((O.unpack_codes(c1) & 7 != 0).sum()) == pages["tile_survivors"]["row_of_large_rowwise_survivors"]


def test_2d_nan_tile_and_nan_amax():
    x = _tensor(32, 32, 10)
    x[20, 3] = np.nan
    c, s, ct, st = O.quantize_2d(x, float(np.nanmax(np.abs(x))))
    assert (s[16:32, 0] == 0x7F).all() and (st[0:16, 1] == 0x7F).all()
    assert (O.unpack_codes(c)[16:32, 0:16] == 0).all()
    assert (s[0:16, 0] != 0x7F).all()
    c, s, ct, st = O.quantize_2d(x, float("nan"))
    assert (s == 0x7F).all() and (st == 0x7F).all() and (c == 0).all() and (ct == 0).all()


def test_2d_ue5m3_transpose_identity():
    x = _tensor(32, 48, 11, spread=3.0)
    c, s, ct, st = O.quantize_2d(x, O.tensor_amax(x), fmt=UE5M3)
    assert np.array_equal(O.unpack_codes(ct), O.unpack_codes(c).T)
