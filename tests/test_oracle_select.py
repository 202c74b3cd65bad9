"""Pins of the oracle's other block-scale selection rules: Four-Over-Six by
the absolute error (MAE) and by the largest error ("Four Over Six"
summaries: Methodologie, Key claims), and the MSE scale sweep over every
scale code ("Scale Learning" blog: scale-setting by MSE initializes the
learned scales).  Checked against the page's vignette, exact rational
arithmetic, brute force over codes, and invariants.  CPU only."""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

E4M3, UE5M3 = O.FMT_E4M3, O.FMT_UE5M3
RULES = [O.SELECT_4OVER6, O.SELECT_4OVER6_MAE, O.SELECT_4OVER6_MAXERR]


def _bf16(x):
    u = np.asarray(x, np.float32).view(np.uint32)
    return (((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16).view(np.float32)


def _blocks(nblocks, seed, spread=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((nblocks, 16)) * np.exp(rng.normal(0, spread, (nblocks, 1)))
    x[rng.random((nblocks, 16)) < 0.05] *= 8
    return _bf16(x.astype(np.float32))


def _unpack(codes):
    out = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
    out[:, 0::2] = codes & 15
    out[:, 1::2] = codes >> 4
    return out


def _exact_errors(xrow, code, alpha, fmt=E4M3):
    """Exact residuals of a block encoded at scale code `code` by the
    oracle's element rule (q = RNE of x * INV_S in binary32), in rationals."""
    D = O.scale_decode(fmt, code)
    S = np.float32(D * alpha)
    inv = np.float32(0.0) if S == 0 else np.float32(1.0) / S
    d = []
    for v in xrow:
        q = O.e2m1_value(O.e2m1_code(np.float32(v) * inv))
        d.append(Fraction(float(v)) - Fraction(float(q)) * Fraction(float(S)))
    return d


# ---------------------------------------------------------------- the page's vignette
def test_vignette_absolute_and_max_error_choose_four(pages):
    """The page's blocks, zero-padded to 16, at alpha = 1.  [10, 20, 30, 40]:
    max->6 picks scale 6.5 and gives x_hat = [9.75, 19.5, 26, 39], residuals
    [0.25, 0.5, 4, 1] (squares 17.3125 = 4 x the printed MSE 4.33; sum 5.75;
    largest 4); max->4 picks 10 and is exact.  [15, 30, 120, 180] is exact
    under max->6 (scale 30).  Every rule makes the page's choice."""
    v = pages["vignette"]
    want6 = {O.SELECT_4OVER6: 17.3125, O.SELECT_4OVER6_MAE: 5.75, O.SELECT_4OVER6_MAXERR: 4.0}
    assert abs(want6[O.SELECT_4OVER6] / 4 - v["blocks"][0]["mse6"]) <= v["mse_print_tolerance"]
    A = np.float32(6 * 448)  # alpha = 1 with S_g = 448
    for blk in v["blocks"]:
        x = np.zeros((1, 16), np.float32)
        x[0, :4] = blk["values"]
        four = blk["choose"] == 4
        for rule in RULES:
            c, s, n4, e_sel, e6 = O.quantize(x, A, select=rule, global_max=448.0, want_sse=True)
            assert n4 == (1 if four else 0), (blk["values"], rule)
            assert e_sel[0, 0] == 0.0
            if four:
                assert O.scale_decode(E4M3, s[0, 0]) == 10.0
                assert e6[0, 0] == want6[rule]
            else:
                assert O.scale_decode(E4M3, s[0, 0]) == 30.0 and e6[0, 0] == 0.0


# ---------------------------------------------------------------- exact rationals
@pytest.mark.parametrize("rule", [O.SELECT_4OVER6_MAE, O.SELECT_4OVER6_MAXERR])
def test_rule_errors_match_exact_rationals(rule):
    """Each block's reported error of both candidates equals the exact
    rational absolute-error sum / largest error of its own codes (within the
    binary32 rounding of the sum), and the choice agrees except within
    rounding of a tie."""
    xb = _blocks(300, 11)
    A = float(np.abs(xb).max())
    alpha = O.alpha(A, 256.0)
    c, s, n4, e_sel, e6 = O.quantize(xb, A, select=rule, want_sse=True)
    c6, s6, _, _, _ = O.quantize(xb, A, select=O.SELECT_6, global_max=256.0, want_sse=True)
    undecided = 0
    for b in range(xb.shape[0]):
        r6 = _exact_errors(xb[b], int(s6[b, 0]), alpha)
        four = s[b, 0] != s6[b, 0] or not np.array_equal(c[b], c6[b])
        ex6 = sum(abs(d) for d in r6) if rule == O.SELECT_4OVER6_MAE else max(abs(d) for d in r6)
        tol = Fraction(float(ex6)) * Fraction(1, 1 << 20) + Fraction(1, 1 << 126)
        assert abs(Fraction(float(e6[b, 0])) - ex6) <= tol
        if four:
            r4 = _exact_errors(xb[b], int(s[b, 0]), alpha)
            ex4 = sum(abs(d) for d in r4) if rule == O.SELECT_4OVER6_MAE else max(abs(d) for d in r4)
            assert abs(Fraction(float(e_sel[b, 0])) - ex4) <= tol
            if ex4 >= ex6:
                undecided += 1  # chosen on a binary32 tie-break of near-equal sums
    assert undecided <= 2


@pytest.mark.parametrize("rule", RULES)
def test_rule_never_worse_than_six(rule):
    xb = _blocks(2000, 12, spread=2.0)
    A = float(np.abs(xb).max())
    c, s, n4, e_sel, e6 = O.quantize(xb, A, select=rule, want_sse=True)
    assert np.all(e_sel <= e6)
    assert 0 < n4 < xb.shape[0]
    assert n4 == int((e_sel < e6).sum())


def test_rules_differ_somewhere():
    """The three rules are different rules: on a varied tensor they choose
    max->4 on different sets of blocks."""
    xb = _blocks(4000, 13, spread=2.0)
    A = float(np.abs(xb).max())
    picks = []
    for rule in RULES:
        c, s, n4 = O.quantize(xb, A, select=rule)
        c6, s6, _ = O.quantize(xb, A, select=O.SELECT_6, global_max=256.0)
        picks.append(s != s6)
    assert not np.array_equal(picks[0], picks[1])
    assert not np.array_equal(picks[0], picks[2])


# ---------------------------------------------------------------- the sweep
def test_sweep_is_the_exact_minimum_over_codes():
    """The sweep's code attains the smallest exact squared error over all 127
    finite E4M3 codes, up to binary32 rounding of the SSE tree."""
    xb = _blocks(40, 21)
    A = float(np.abs(xb).max())
    alpha = O.alpha(A, 448.0)
    c, s, _, e_sel, _ = O.quantize(xb, A, select=O.SELECT_SWEEP, want_sse=True)
    for b in range(xb.shape[0]):
        exact = [sum(d * d for d in _exact_errors(xb[b], code, alpha)) for code in range(0x7F)]
        best = min(exact)
        got = exact[int(s[b, 0])]
        assert got - best <= best * Fraction(1, 1 << 19) + Fraction(1, 1 << 140)
        assert abs(Fraction(float(e_sel[b, 0])) - got) <= got * Fraction(1, 1 << 20) + Fraction(1, 1 << 140)


def test_sweep_never_worse_than_either_four_over_six_candidate():
    """Both Four-Over-Six candidates are among the swept codes and their SSE
    is computed by the same tree: the sweep's SSE is at most either."""
    xb = _blocks(3000, 22, spread=2.0)
    A = float(np.abs(xb).max())
    _, _, _, e_sw, e6 = O.quantize(xb, A, select=O.SELECT_SWEEP, global_max=256.0, want_sse=True)
    _, _, _, e46, _ = O.quantize(xb, A, select=O.SELECT_4OVER6, global_max=256.0, want_sse=True)
    assert np.all(e_sw <= e46) and np.all(e_sw <= e6)
    assert (e_sw < e46).mean() > 0.2


def test_sweep_zero_and_representable_blocks():
    """A zero block keeps code 0; a block of exact NVFP4 values (alpha a power
    of two) is reproduced exactly by the code the sweep picks."""
    A = 6.0 * 448.0 * 2.0 ** -4
    x = np.zeros((3, 16), np.float32)
    D = O.scale_decode(E4M3, 0x55)
    x[1] = np.array([6, -4, 3, 0.5, 1, 1.5, 2, 0, -6, 4, 3, 2, 1, 0.5, -0.5, 6]) * D * 2.0 ** -4
    x[2] = np.array([3, 1, 0.5, 0, 2, 1.5, 1, 3, 3, 2, 1, 0, 0.5, 1, 1.5, 2]) * D * 2.0 ** -4
    c, s, _, e, _ = O.quantize(x, A, select=O.SELECT_SWEEP, global_max=448.0, want_sse=True)
    assert s[0, 0] == 0 and np.all(c[0] == 0) and e[0, 0] == 0
    xh = O.dequantize(c, s, A, global_max=448.0)
    assert np.array_equal(xh[1:], x[1:]) and np.all(e[1:] == 0)


def test_sweep_ue5m3_and_2d_shapes():
    xb = _blocks(64, 23).reshape(8, 128)
    A = float(np.abs(xb).max())
    c, s, _, e_sw, _ = O.quantize(xb, A, fmt=UE5M3, select=O.SELECT_SWEEP, want_sse=True)
    _, _, _, e46, _ = O.quantize(xb, A, fmt=UE5M3, select=O.SELECT_4OVER6,
                                 global_max=114688.0, want_sse=True)
    assert np.all(e_sw <= e46)
    with pytest.raises(ValueError):
        O.quantize(xb, A, select=O.SELECT_SWEEP, rounding=O.ROUND_SR)
