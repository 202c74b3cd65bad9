"""Pins of the oracle's quantizer (block scaling, Four-Over-Six, stochastic
rounding, dequantization) against the pages' worked values, invariants the
method guarantees, and brute force over every scale code with exact rational
arithmetic.  CPU only."""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

E4M3 = O.FMT_E4M3
A_UNIT_448 = 6.0 * 448.0  # tensor amax that makes alpha exactly 1 (S_g = 448)
A_UNIT_256 = 6.0 * 256.0  # same under the Four-Over-Six default S_g = 256


def _block(vals):
    x = np.zeros((1, 16), np.float32)
    x[0, :len(vals)] = vals
    return x


def _q1(x, amax, **kw):
    codes, scales, n4 = O.quantize(x, amax, **kw)
    return O.unpack_codes(codes), scales, n4


def test_block_max_54(pages):
    ex = pages["block_max_54"]
    x = _block([ex["block_max"], 3.0, -1.0, 0.0])
    nib, sc, _ = _q1(x, A_UNIT_448, select=O.SELECT_6)
    assert O.scale_decode(E4M3, sc[0, 0]) == ex["scale"]
    assert O.e2m1_value(nib[0, 0]) == ex["value"]


def test_widget_576(pages):
    ex = pages["widget_576"]
    x = _block([ex["input"]])
    codes, sc, _ = O.quantize(x, A_UNIT_448, select=O.SELECT_6)
    assert O.scale_decode(E4M3, sc[0, 0]) == ex["scale"]
    assert O.e2m1_value(O.unpack_codes(codes)[0, 0]) == ex["value"]
    xhat = O.dequantize(codes, sc, A_UNIT_448, select=O.SELECT_6)
    assert xhat[0, 0] == ex["reconstructed"]
    assert round(float(x[0, 0]) - float(xhat[0, 0]), 1) == ex["error"]


def test_nvfp4_extremes(pages):
    r = pages["nvfp4_range"]
    # the largest representable magnitude at alpha = 1 and at alpha = 2
    for amax, top in [(A_UNIT_448, r["max"]), (2 * A_UNIT_448, r["alpha2_max"])]:
        x = _block([top, -top / 6 * 0.5])
        codes, sc, _ = O.quantize(x, amax, select=O.SELECT_6)
        xh = O.dequantize(codes, sc, amax, select=O.SELECT_6)
        assert xh[0, 0] == top
    # the smallest: 0.5 x smallest E4M3 subnormal (block max 2^-10 -> scale
    # ~1.67e-4 rounds to 2^-9... the element itself maps to code 1 = 0.5)
    for amax, bot in [(A_UNIT_448, r["min"]), (2 * A_UNIT_448, r["alpha2_min"])]:
        alpha = O.alpha(amax, 448.0)
        codes = np.array([[0x01] + [0] * 7], np.uint8)  # element 0 = +0.5
        sc = np.array([[0x01]], np.uint8)  # smallest E4M3 subnormal
        xh = O.dequantize(codes, sc, amax, select=O.SELECT_6)
        assert xh[0, 0] == bot and alpha in (1.0, 2.0)


def test_sr_example(pages):
    ex = pages["sr_requant"]
    # forward: 5.4 in a block whose scale is 9 (block max 54, alpha = 1)
    x = _block([54.0, ex["x"]])
    codes, sc, _ = O.quantize(x, A_UNIT_448, select=O.SELECT_6)
    assert O.scale_decode(E4M3, sc[0, 0]) == ex["scale_fwd"]
    assert O.e2m1_value(O.unpack_codes(codes)[0, 1]) == ex["code_value_fwd"]
    assert O.dequantize(codes, sc, A_UNIT_448, select=O.SELECT_6)[0, 1] == ex["reconstructed"]
    # backward: 4.5 at scale 2 is 2.25 -> 2 w.p. 3/4, 3 w.p. 1/4
    y = np.float32(ex["reconstructed"] / ex["scale_bwd"])
    assert y == ex["y_bwd"]
    n = 200000
    vals = np.array([O.e2m1_value(O.e2m1_code_sr(float(y), O.sr_hash(1234, i))) for i in range(n)])
    assert set(np.unique(vals)) == {ex["lo"], ex["hi"]}
    frac = float((vals == ex["hi"]).mean())
    sigma = np.sqrt(ex["p_hi"] * (1 - ex["p_hi"]) / n)
    assert abs(frac - ex["p_hi"]) < 5 * sigma
    assert abs(ex["scale_bwd"] * vals.mean() - ex["reconstructed"]) < 5 * sigma * ex["scale_bwd"]


def test_sr_threshold_makes_it_unbiased():
    """Up iff u + F >= 2^22 with u = h >> 10 uniform on 22 bits and F the
    fraction truncated to 22 bits: exactly F of the 2^22 variates round up, so
    E[q] = |y| whenever p has at most 22 fractional bits (every |y| >= 1) and
    falls short by less than 2^-22 of a step otherwise."""
    rng = np.random.default_rng(5)
    ys = np.concatenate([rng.uniform(0.25, 6.0, 300).astype(np.float32),
                         rng.uniform(1e-6, 0.25, 100).astype(np.float32),
                         np.array([0.25, 0.3, 1.1, 2.25, 4.5, 5.999999, 1e-30], np.float32)])
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for y in ys:
        a = Fraction(float(y))
        lo = max(g for g in grid if g <= a)
        hi = min(g for g in grid if g > a)
        step = Fraction(hi) - Fraction(lo)
        p = (a - Fraction(lo)) / step
        F = int(p * 2 ** 22)  # floor
        T = 2 ** 22 - F        # smallest u that rounds up
        if T <= 2 ** 22 - 1:
            assert O.e2m1_value(O.e2m1_code_sr(float(y), T << 10)) == hi
            assert O.e2m1_value(O.e2m1_code_sr(float(y), (T << 10) | 0x3FF)) == hi
        if T >= 1:
            assert O.e2m1_value(O.e2m1_code_sr(float(y), (T - 1) << 10)) == lo
            assert O.e2m1_value(O.e2m1_code_sr(float(y), ((T - 1) << 10) | 0x3FF)) == lo
        # expectation over the 2^22 variates
        e = Fraction(lo) + step * Fraction(F, 2 ** 22)
        assert e <= a and a - e < step * Fraction(1, 2 ** 22)
        if a >= 1:
            assert e == a
    # on-grid values never move, and the sign is kept
    for g in grid:
        for h in (0, 0xFFFFFFFF, 0x12345678):
            assert O.e2m1_value(O.e2m1_code_sr(g, h)) == g
            assert O.e2m1_value(O.e2m1_code_sr(-g, h)) == -g


def test_four_over_six_fractions(pages):
    ex = pages["four_over_six_fractions"]
    # block max 40 with scale 10 exactly representable (max->4: 40/4 = 10)
    m = 40.0
    x = _block([m, ex["frac_exact_3_at_scale4"] * m])
    nib6, sc6, _ = _q1(x, A_UNIT_256, select=O.SELECT_6, global_max=256.0)
    nib46, sc46, n4 = _q1(x, A_UNIT_256, select=O.SELECT_4OVER6)
    assert O.scale_decode(E4M3, sc46[0, 0]) == 10.0 and n4 == 1
    assert O.e2m1_value(nib46[0, 1]) == 3.0  # 75% of the max is exactly 3
    # max->6 of a max of 48 (scale 8 exact): code 4 sits at 2/3 of the max
    x = _block([48.0, 48.0 * ex["frac_code4_at_scale6"], 0.75 * 48.0])
    nib6, sc6, _ = _q1(x, A_UNIT_256, select=O.SELECT_6, global_max=256.0)
    assert O.scale_decode(E4M3, sc6[0, 0]) == 8.0
    assert O.e2m1_value(nib6[0, 1]) == 4.0
    assert O.e2m1_value(nib6[0, 2]) == 4.0  # 75% -> y = 4.5 -> 4 (RNE)


def test_vignette(pages):
    v = pages["vignette"]
    for blk in v["blocks"]:
        x = _block(blk["values"])
        _, sc6, _, _, e6 = O.quantize(x, A_UNIT_256, select=O.SELECT_6, global_max=256.0,
                                      want_sse=True)
        _, sc46, n4, esel, _ = O.quantize(x, A_UNIT_256, select=O.SELECT_4OVER6, want_sse=True)
        mse6 = float(e6[0, 0]) / len(blk["values"])
        assert abs(mse6 - blk["mse6"]) <= v["mse_print_tolerance"]
        assert n4 == (1 if blk["choose"] == 4 else 0)
        if "mse4" in blk:
            assert float(esel[0, 0]) / len(blk["values"]) == blk["mse4"]


def test_range_loss(pages):
    r = pages["range_loss_256"]
    assert round(100 * (1 - r["fp8_max_four_over_six"] / r["fp8_max_default"]), 1) == r["range_loss_percent"]
    # with S_g = 256 the block holding the tensor max gets a max->4 scale of
    # 256 * 1.5 = 384 <= 448: no saturation of the E4M3 scale
    x = _block([100.0, 7.0])
    amax = 100.0
    kq4 = np.float32(1.0) / (np.float32(4.0) * np.float32(O.alpha(amax, 256.0)))
    s_raw = np.float32(np.float32(100.0) * kq4)
    assert abs(float(s_raw) - r["fp8_max_four_over_six"] * r["scale_ratio"]) < 1e-3
    assert O.scale_encode(E4M3, float(s_raw)) < 0x7E


def test_tile_survivors(pages):
    t = pages["tile_survivors"]
    rng = np.random.default_rng(0)
    small = rng.uniform(0.5, 1.5, (16, 16)).astype(np.float32)
    tile = small.copy()
    tile[5, :] = 1000.0  # a full row of large values
    amax = 1000.0
    codes, _, _ = O.quantize(tile, amax, select=O.SELECT_6)
    assert int((O.unpack_codes(codes) & 7 != 0).sum()) == t["row_of_large_rowwise_survivors"]
    codes_t, _, _ = O.quantize_cols(tile, amax, select=O.SELECT_6)
    assert int((O.unpack_codes(codes_t) & 7 != 0).sum()) < 128  # most small values flush
    tile = small.copy()
    tile[7, 3] = 1000.0  # one outlier
    codes, _, _ = O.quantize(tile, amax, select=O.SELECT_6)
    assert int((O.unpack_codes(codes) & 7 != 0).sum()) == t["one_outlier_rowwise_survivors"]


# ---------------------------------------------------------------- invariants
def _random_tensor(rows, cols, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)) * np.exp(rng.normal(0, 1.5, (rows, 1)))
    x[rng.random((rows, cols)) < 0.01] *= 30
    x = x.astype(np.float32)
    # round to bf16 so that the oracle sees the same values the GPU would
    u = x.view(np.uint32)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return u


@pytest.mark.parametrize("select", [O.SELECT_6, O.SELECT_4OVER6])
def test_quantize_invariants(select):
    xb = _random_tensor(64, 256, 1)
    x = O.as_f32(xb)
    amax = O.tensor_amax(xb)
    sg = O.default_global_max(E4M3, select)
    codes, sc, n4, esel, e6 = O.quantize(xb, amax, select=select, want_sse=True)
    B = sc.size
    assert 0 <= n4 <= B
    if select == O.SELECT_6:
        assert n4 == 0 and np.array_equal(esel, e6)
    assert np.all(esel <= e6)
    assert np.all(sc <= 0x7E)
    xh, bs = O.dequantize(codes, sc, amax, select=select, want_block_scale=True)
    # |x_hat| <= 6 s: the clamp at q_max; x_hat is the correctly rounded
    # q * D * alpha, so the bound is the rounded 6 * D * alpha
    D = np.vectorize(lambda c: O.scale_decode(E4M3, int(c)))(sc)
    lim = (6.0 * D * float(O.alpha(amax, sg))).astype(np.float32)
    assert np.all(np.abs(xh) <= np.repeat(lim, 16, axis=1))
    # the tensor amax block gets (close to) S_g as its max->6 scale
    alpha = O.alpha(amax, sg)
    assert bs.max() <= 1.5 * sg * alpha * (1 + 2 ** -3)
    # SSE from the dequantized tensor agrees with the per-block SSE bookkeeping
    tot = O.sse(x, xh)
    assert abs(tot - float(esel.astype(np.float64).sum())) <= 1e-4 * tot


def test_idempotent_on_representable_values():
    rng = np.random.default_rng(2)
    for k in (-3, 0, 4):
        amax_alpha = 2.0 ** k  # alpha
        rows = 32
        q = rng.choice([-6, -4, -3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3, 4, 6], (rows, 16))
        q[:, 0] = np.where(rng.random(rows) < 0.5, 6.0, -6.0)  # block max |q| = 6
        c = rng.integers(0x08, 0x7E, rows)
        D = np.array([O.scale_decode(E4M3, int(ci)) for ci in c])
        x = (q * D[:, None] * amax_alpha).astype(np.float32)
        A = float(np.abs(x).max())
        # choose S_g so that alpha == 2^k exactly: alpha = A / (6 S_g)
        sg = A / (6.0 * amax_alpha)
        assert O.alpha(A, sg) == amax_alpha
        for select in (O.SELECT_6, O.SELECT_4OVER6):
            codes, sc, n4 = O.quantize(x, A, select=select, global_max=sg)
            nib = O.unpack_codes(codes)
            if select == O.SELECT_6:
                assert np.array_equal(sc[:, 0], c)
                assert np.array_equal(np.vectorize(O.e2m1_value)(nib), q)
            xh = O.dequantize(codes, sc, A, select=select, global_max=sg)
            assert np.array_equal(xh, x)
            assert n4 == 0


def _exact_sse(xrow, nib, D, alpha):
    a = Fraction(float(alpha))
    s = Fraction(0)
    for xi, n in zip(xrow, nib):
        d = Fraction(float(xi)) - Fraction(O.e2m1_value(int(n))) * Fraction(float(D)) * a
        s += d * d
    return s


def _exact_rne_codes(xrow, D, alpha):
    """E2M1 RNE of the exact rational x / (D alpha), brute force."""
    grid = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
            Fraction(4), Fraction(6)]
    out = []
    for xi in xrow:
        y = Fraction(float(xi)) / (Fraction(float(D)) * Fraction(float(alpha)))
        a = abs(y)
        best = min(range(8), key=lambda k: (abs(a - grid[k]), k & 1))
        out.append(best | (8 if float(xi) < 0 or (float(xi) == 0 and np.signbit(xi)) else 0))
    return out


def test_brute_force_over_all_scale_codes():
    """On small blocks: the exact-rational SSE of the oracle's 4/6 result is no
    larger than its scale-6 result, and no smaller than the best over every
    nonzero E4M3 scale code; element codes equal exact RNE of x / s except
    within binary32 rounding of a midpoint."""
    rng = np.random.default_rng(9)
    nblk = 60
    xb = _random_tensor(nblk, 16, 4)
    x = O.as_f32(xb)
    amax = float(O.tensor_amax(xb))
    alpha = O.alpha(amax, 256.0)
    codes, sc, n4, esel, e6 = O.quantize(xb, amax, select=O.SELECT_4OVER6, want_sse=True)
    codes6, sc6, _ = O.quantize(xb, amax, select=O.SELECT_6, global_max=256.0)
    nib, nib6 = O.unpack_codes(codes), O.unpack_codes(codes6)
    dec = [O.scale_decode(E4M3, c) for c in range(0x7F)]
    near_ties = 0
    elem_mismatch = 0
    for b in range(nblk):
        s46 = _exact_sse(x[b], nib[b], dec[sc[b, 0]], alpha)
        s6 = _exact_sse(x[b], nib6[b], dec[sc6[b, 0]], alpha)
        best = min(_exact_sse(x[b], _exact_rne_codes(x[b], dec[c], alpha), dec[c], alpha)
                   for c in range(1, 0x7F))
        assert best <= s46
        if s46 > s6:
            # only possible when the binary32 SSEs are within rounding of a tie
            near_ties += 1
            assert float(s46 - s6) <= 1e-5 * float(s6)
        exact = _exact_rne_codes(x[b], dec[sc[b, 0]], alpha)
        elem_mismatch += sum(int(a != e) for a, e in zip(nib[b], exact))
    assert near_ties <= 1
    assert elem_mismatch <= 2


def test_scale_six_matches_pages_formula_on_scale_codes():
    """a_b * K_6 encodes to the same E4M3 code as the exact a_b / (6 alpha)
    except within binary32 rounding of an E4M3 midpoint."""
    xb = _random_tensor(256, 64, 6)
    x = O.as_f32(xb)
    amax = float(O.tensor_amax(xb))
    alpha = O.alpha(amax, 448.0)
    _, sc, _ = O.quantize(xb, amax, select=O.SELECT_6)
    amax_b = np.abs(x.reshape(-1, 16)).max(axis=1)
    ref = np.array([O.scale_encode(E4M3, float(np.float32(Fraction(float(a)) / (6 * Fraction(float(alpha))))))
                    for a in amax_b])
    assert int((ref != sc.ravel()).sum()) <= 2


def test_nan_amax_gives_nan_scales():
    xb = _random_tensor(4, 32, 8)
    for bad in (float("nan"), float("inf"), -1.0):
        codes, sc, n4 = O.quantize(xb, bad, select=O.SELECT_4OVER6)
        assert np.all(sc == 0x7F) and np.all(codes == 0) and n4 == 0
        assert np.all(np.isnan(O.dequantize(codes, sc, 1.0)))
    codes, sc, _ = O.quantize(xb, float("nan"), fmt=O.FMT_UE5M3, select=O.SELECT_6)
    assert np.all(sc == 0xFF)


def test_zero_tensor_and_zero_blocks():
    x = np.zeros((2, 32), np.float32)
    x[1, 16:] = -0.0
    codes, sc, n4 = O.quantize(x, 0.0)
    assert O.alpha(0.0, 256.0) == 1.0
    assert np.all(sc == 0) and n4 == 0
    nib = O.unpack_codes(codes)
    assert np.all(nib[0] == 0) and np.all(nib[1, :16] == 0) and np.all(nib[1, 16:] == 8)
    xh = O.dequantize(codes, sc, 0.0)
    assert np.all(xh == 0)


def test_reciprocal_overflow_of_tiny_amax():
    """A tensor amax so small that 1 / (6 alpha) overflows binary32: the
    per-tensor constant K_6 is then the largest finite float, not infinity
    (the oracle's reading of an overflowing reciprocal), so a block holding the
    tensor maximum A = 2^-123 gets the scale code nearest to fl(A * FLT_MAX)
    = 31.999998 (E4M3 32 = 0x60) instead of saturating at 448, and a block
    whose maximum is A / 4 gets the code nearest to 8 (0x50)."""
    A = np.float32(2.0 ** -123)
    alpha = A / np.float32(6.0 * 448.0)
    with np.errstate(over="ignore"):
        assert np.isinf(np.float32(1.0) / (np.float32(6.0) * alpha))
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = A
    x[0, 16] = A / 4
    kmax = np.finfo(np.float32).max
    want = [O.scale_encode(E4M3, float(np.float32(A) * kmax)),
            O.scale_encode(E4M3, float(np.float32(A / 4) * kmax))]
    assert want == [0x60, 0x50]
    for select in (O.SELECT_6, O.SELECT_4OVER6):
        _, scales, _ = _q1(x, float(A), select=select, global_max=448.0)
        assert list(scales[0]) == want, select


def test_sr_rejected_with_four_over_six():
    with pytest.raises(ValueError):
        O.quantize(np.zeros((1, 16), np.float32), 1.0, select=O.SELECT_4OVER6, rounding=O.ROUND_SR)
    with pytest.raises(ValueError):
        O.quantize(np.zeros((1, 8), np.float32), 1.0)


def test_sr_index_orientation():
    """Row-wise SR hashes r*C + c; column-wise hashes c*R + r (the index in
    the transposed output), so the two passes draw independent variates."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((32, 48)).astype(np.float32)
    amax = float(np.abs(x).max())
    codes, sc, _ = O.quantize(x, amax, fmt=O.FMT_UE5M3, select=O.SELECT_6,
                              rounding=O.ROUND_SR, seed=1234)
    # element (r, c) recomputed one at a time
    alpha = O.alpha(amax, 114688.0)
    nib = O.unpack_codes(codes)
    for (r, c) in [(0, 0), (3, 17), (31, 47)]:
        D = O.scale_decode(O.FMT_UE5M3, sc[r, c // 16])
        S = np.float32(np.float32(D) * np.float32(alpha))
        y = np.float32(x[r, c] * np.float32(np.float32(1.0) / S))
        assert nib[r, c] == O.e2m1_code_sr(float(y), O.sr_hash(1234, r * 48 + c))
    ct, st, _ = O.quantize_cols(x, amax, fmt=O.FMT_UE5M3, select=O.SELECT_6,
                                rounding=O.ROUND_SR, seed=1234)
    nibt = O.unpack_codes(ct)
    for (r, c) in [(0, 0), (17, 3), (31, 47)]:
        D = O.scale_decode(O.FMT_UE5M3, st[c, r // 16])
        S = np.float32(np.float32(D) * np.float32(alpha))
        y = np.float32(x[r, c] * np.float32(np.float32(1.0) / S))
        assert nibt[c, r] == O.e2m1_code_sr(float(y), O.sr_hash(1234, c * 32 + r))


def test_nan_and_inf_elements_with_finite_amax():
    x = np.ones((1, 48), np.float32)
    x[0, 3] = np.nan
    x[0, 20] = np.inf
    x[0, 40] = -np.inf
    codes, sc, n4 = O.quantize(x, 10.0, select=O.SELECT_4OVER6)
    nib = O.unpack_codes(codes)
    assert sc[0, 0] == 0x7F and np.all(nib[0, :16] == 0)
    assert sc[0, 1] == 0x7E and nib[0, 20] == 7 and n4 == 0
    assert sc[0, 2] == 0x7E and nib[0, 40] == 15
