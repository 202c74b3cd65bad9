"""Pins of the oracle's re-quantization for the backward pass ("End-to-End
4-Bit Training", 'Re-quantization with stochastic rounding': dequantize the
forward tensor, transpose it in higher precision, re-quantize it with
stochastic rounding to NVFP4 or MXFP8) against the page's worked example,
unbiasedness, exact identities on representable values, and the MXFP8 block
rules (OCP Microscaling: blocks of 32, power-of-two E8M0 scale, E4M3
elements).  CPU only."""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

E4M3, UE5M3 = O.FMT_E4M3, O.FMT_UE5M3
SCALE_9, SCALE_2, SCALE_448 = 0x51, 0x40, 0x7E  # E4M3 bytes of 9.0, 2.0, 448


def _pack(nibbles):
    """[rows, cols] nibbles -> NVFP4 code bytes (even column in the low nibble)."""
    n = np.asarray(nibbles, np.uint8)
    return (n[:, 0::2] | (n[:, 1::2] << 4)).astype(np.uint8)


def _unpack(codes):
    c = np.asarray(codes, np.uint8)
    out = np.empty((c.shape[0], c.shape[1] * 2), np.uint8)
    out[:, 0::2] = c & 15
    out[:, 1::2] = c >> 4
    return out


def _nvfp4_values(codes, scales, alpha):
    """Exact values of an NVFP4 tensor in float64 (q * D * alpha)."""
    q = np.vectorize(O.e2m1_value)(_unpack(codes)).astype(np.float64)
    d = np.vectorize(lambda c: O.scale_decode(E4M3, c))(scales).astype(np.float64)
    return q * np.repeat(d, 16, axis=1) * alpha


def _page_example_source(pages, cols):
    """16 x cols NVFP4 tensor with alpha = 1 (A = 6 * 448): row 0 holds the
    page's forward value (0.5 at block scale 9 -> 4.5) in every column; row 1
    holds 12 = 6 * 2 in every column, so each column block's amax is 12 and
    its new scale 12 / 6 = 2, the page's backward scale."""
    ex = pages["sr_requant"]
    assert O.scale_decode(E4M3, SCALE_9) == ex["scale_fwd"]
    assert O.scale_decode(E4M3, SCALE_2) == ex["scale_bwd"]
    nib = np.zeros((16, cols), np.uint8)
    nib[0, :] = O.e2m1_code(ex["code_value_fwd"])       # 0.5
    nib[1, :] = O.e2m1_code(6.0)
    scales = np.zeros((16, cols // 16), np.uint8)
    scales[0, :] = SCALE_9
    scales[1, :] = SCALE_2
    return _pack(nib), scales, 6.0 * 448.0


def test_page_example_reconstruction(pages):
    ex = pages["sr_requant"]
    # forward: 5.4 / 9 = 0.6 -> nearest E2M1 0.5 -> 4.5
    assert O.e2m1_value(O.e2m1_code(np.float32(ex["x"]) / np.float32(ex["scale_fwd"]))) == ex["code_value_fwd"]
    codes, scales, A = _page_example_source(pages, 32)
    xh = O.dequantize(codes, scales, A, global_max=448.0)
    assert np.all(xh[0] == ex["reconstructed"]) and np.all(xh[1] == 12.0)
    assert O.dequantized_amax(codes, scales, amax=A, global_max=448.0) == 12.0


def test_page_example_sr_frequencies(pages):
    """4.5 re-quantized at scale 2 is 2.25: 2 with probability 3/4, 3 with
    probability 1/4, 4.5 in expectation (binomial test over 4096 columns,
    each with its own element index, and a second seed)."""
    ex = pages["sr_requant"]
    cols = 4096
    codes, scales, A = _page_example_source(pages, cols)
    for seed in (1234, 99):
        ct, st = O.requant_t(codes, scales, amax=A, global_max=448.0, target="nvfp4",
                             dst_amax=A, dst_global_max=448.0, seed=seed)
        assert np.all(st[:, 0] == SCALE_2)                       # the page's backward scale
        q = np.vectorize(O.e2m1_value)(_unpack(ct)[:, 0])         # transposed row c, element 0
        assert set(np.unique(q)) <= {ex["lo"], ex["hi"]}
        n_hi = int((q == ex["hi"]).sum())
        sd = np.sqrt(cols * ex["p_hi"] * (1 - ex["p_hi"]))
        assert abs(n_hi - cols * ex["p_hi"]) < 5 * sd
        mean = 2.0 * q.mean()
        assert abs(mean - ex["reconstructed"]) < 5 * 2.0 * sd / cols
        # the 12s are on the grid at scale 2 (value 6): never moved
        assert np.all(_unpack(ct)[:, 1] == O.e2m1_code(6.0))


def test_page_example_mxfp8(pages):
    """The page notes that SR on dequantized values allows any target
    precision: to MXFP8 the 4.5 and the 12 of each column are exact (E4M3
    holds them at the block's power-of-two scale), so no element moves."""
    codes, scales, A = _page_example_source(pages, 64)
    codes = np.concatenate([codes, np.zeros_like(codes)])        # 32 rows: one MXFP8 block
    scales = np.concatenate([scales, np.zeros_like(scales)])
    el, sc = O.requant_t(codes, scales, amax=A, global_max=448.0, target="mxfp8", seed=5)
    assert el.shape == (64, 32) and sc.shape == (64, 1)
    # amax 12 = 1.5 * 2^3 -> e = 3 - 8 = -5: 12 * 2^5 = 384, 4.5 * 2^5 = 144
    assert np.all(sc == 127 - 5)
    d = O.mxfp8_dequantize(el, sc)
    assert np.all(d[:, 0] == 4.5) and np.all(d[:, 1] == 12.0) and np.all(d[:, 2:] == 0.0)


# ---------------------------------------------------------------- unbiasedness
def _random_source(rows, cols, seed, per_row=False):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * np.exp(rng.normal(0, 1.0, (rows, 1)))).astype(np.float32)
    if per_row:
        ra = O.row_amax(x)
        c, s, _ = O.quantize_rowscaled(x, ra, select=O.SELECT_4OVER6)
        return c, s, dict(row_amaxes=ra)
    A = O.tensor_amax(x)
    c, s, _ = O.quantize(x, A, select=O.SELECT_4OVER6)
    return c, s, dict(amax=A)


def _steps(xt, ct, st, target, alpha2):
    """Grid step (in x units) at each element of the transposed tensor, and
    whether the element lies inside its block's range (|y| <= 6, or <= 448
    for MXFP8).  Elements outside saturate in every draw: the clipping of a
    block maximum whose scale was rounded down, not a property of SR."""
    ax = np.abs(xt)
    if target == "nvfp4":
        S = np.repeat(np.vectorize(lambda c: O.scale_decode(E4M3, c))(st), 16, axis=1) * alpha2
        y = ax / S
        step = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0)) * S
        return step, y <= 6.0
    X = np.repeat(2.0 ** (st.astype(np.float64) - 127), 32, axis=1)
    y = ax / X
    e = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
    step = np.where(y < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - 3)) * X
    return step, y <= 448.0


@pytest.mark.parametrize("target", ["nvfp4", "mxfp8"])
@pytest.mark.parametrize("per_row", [False, True])
def test_requant_is_unbiased(target, per_row):
    """E over seeds of the re-quantized tensor is the transposed dequantized
    tensor ([E2E]: forward and backward tensors equal in expectation), for
    every element inside its block's range.  A wrong transpose, block scale
    or outer scale moves the mean by whole grid steps."""
    rows, cols, nseed = 32, 48, 400
    codes, scales, src = _random_source(rows, cols, 7, per_row)
    xh = (O.dequantize_rowscaled(codes, scales, src["row_amaxes"]) if per_row
          else O.dequantize(codes, scales, src["amax"]))
    xt = xh.T.astype(np.float64)
    A2 = O.dequantized_amax(codes, scales, **src)
    assert A2 == np.abs(xh).max()
    acc = np.zeros_like(xt)
    st0 = None
    for seed in range(nseed):
        ct, st = O.requant_t(codes, scales, **src, target=target, dst_amax=A2, seed=seed)
        if st0 is None:
            st0 = st
        assert np.array_equal(st, st0)          # the scales do not depend on the seed
        if target == "nvfp4":
            v = _nvfp4_values(ct, st, O.alpha(A2, 448.0))
        else:
            v = O.mxfp8_dequantize(ct, st).astype(np.float64)
        acc += v
    mean = acc / nseed
    step, inside = _steps(xt, ct, st0, target, O.alpha(A2, 448.0))
    assert inside.mean() > 0.95
    # per element: within 6 standard deviations of a draw's mean (sd <= step/2)
    err = np.abs(mean - xt)
    assert np.all(err[inside] <= 6 * 0.5 * step[inside] / np.sqrt(nseed) + 1e-9 * step[inside])
    # aggregate: the signed errors in units of the step average out
    z = ((mean - xt) / step)[inside]
    assert abs(z.mean()) < 6 * 0.5 / np.sqrt(nseed * z.size)
    # the saturated block maxima are clipped to 6 S (448 X), below |x_hat|
    assert np.all(err[~inside] > 0)


# ---------------------------------------------------------------- exact identities
def _tiled_source(rows, cols, seed, k=-3):
    """16x16-tile-scaled tensor whose every row block and column block holds
    the tile's largest magnitude 6 * D * alpha (a signed permutation pattern
    of 6s in each tile).  alpha = 2^k (the amax passed is 6 * 448 * 2^k) and
    the tile scales D are powers of two, so x / (D alpha) is exactly q."""
    rng = np.random.default_rng(seed)
    A = 6.0 * 448.0 * 2.0 ** k                       # alpha = 2^k under S_g = 448
    x = np.zeros((rows, cols), np.float64)
    for ti in range(rows // 16):
        for tj in range(cols // 16):
            D = 2.0 ** int(rng.integers(-9, 9))     # E4M3 holds 2^-9 .. 2^8 exactly
            q = rng.choice([0, 0.5, 1, 1.5, 2, 3, 4, 6], size=(16, 16)) * rng.choice([-1, 1], size=(16, 16))
            perm = rng.permutation(16)
            q[np.arange(16), perm] = 6.0 * rng.choice([-1, 1], size=16)
            x[ti * 16:(ti + 1) * 16, tj * 16:(tj + 1) * 16] = q * D * 2.0 ** k
    return x.astype(np.float32), A


def test_requant_of_tile_scaled_values_is_their_transpose():
    """With every column block holding its tile's max, the re-quantized
    column blocks get the tile's scale back and every element lands on the
    grid: stochastic rounding moves nothing, and the output is the 16x16
    tile quantizer's own transposed layout bit for bit (w_q = (w_q^T)^T)."""
    x, A = _tiled_source(64, 96, 3)
    codes, scales, codes_t, scales_t = O.quantize_2d(x, A, global_max=448.0)
    for seed in (0, 1, 77):
        ct, st = O.requant_t(codes, scales, amax=A, global_max=448.0, target="nvfp4",
                             dst_amax=A, dst_global_max=448.0, seed=seed)
        assert np.array_equal(st, scales_t)
        assert np.array_equal(ct, codes_t)


def test_mxfp8_on_grid_values_are_kept():
    """Values that are E4M3 numbers times the block's own power of two (block
    max in [256, 448] times 2^e) are returned unchanged under any seed."""
    rng = np.random.default_rng(11)
    grid = np.array([O.scale_decode(E4M3, c) for c in range(0x7F)])
    rows, cols = 8, 128
    e = rng.integers(-20, 20, size=(rows, cols // 32))
    vals = rng.choice(grid, size=(rows, cols)) * rng.choice([-1, 1], size=(rows, cols))
    top = rng.choice(grid[(grid >= 256) & (grid <= 448)], size=(rows, cols // 32))
    vals[:, ::32] = top
    x = (vals * np.repeat(2.0 ** e, 32, axis=1)).astype(np.float32)
    for seed in (0, 5):
        el, sc = O.mxfp8_quantize_sr(x, seed=seed)
        assert np.array_equal(sc.astype(int) - 127, e)
        assert np.array_equal(O.mxfp8_dequantize(el, sc), x)


def test_mxfp8_scale_places_block_max_in_top_binades_and_saturates():
    """The block max lands in [256, 512) after scaling; above 448 it
    saturates to 448 (0x7E), never to NaN; zero blocks get the smallest scale."""
    x = np.zeros((4, 32), np.float32)
    x[0, 3] = 500.0          # e = 0: 500 -> saturates to 448
    x[1, 0] = 0.75           # 0.75 = 1.5 * 2^-1: e = -9, 0.75 * 2^9 = 384 exact
    x[1, 1] = -2.0 ** -20    # far below the block's smallest step: 0 (kept sign)
    x[2, :] = 1e-30          # tiny block: e = floor(log2(1e-30)) - 8 = -108
    el, sc = O.mxfp8_quantize_sr(x, seed=1)
    assert sc[0, 0] == 127 and el[0, 3] == 0x7E
    assert sc[1, 0] == 127 - 9 and O.scale_decode(E4M3, el[1, 0]) * 2.0 ** -9 == 0.75
    assert el[1, 1] in (0x80, 0x81)
    assert sc[2, 0] == 127 - 108
    assert sc[3, 0] == 0 and np.all(el[3] == 0)
    y = 1e-30 * 2.0 ** 108
    assert 256 <= y < 512


def test_e4m3_sr_rule_counts_exactly():
    """Over all 2^20 variates u = h >> 12 the rule rounds up exactly
    floor(p * 2^20) times: P(up) = p for p with at most 20 fractional bits
    (unbiased), and values on the grid never move."""
    for y, lo, hi in [(2.25, 2.25, 2.5), (2.3125, 2.25, 2.5), (100.0, 96.0, 104.0),
                      (0.0029296875, 0.001953125, 0.00390625), (447.0, 416.0, 448.0)]:
        p = (y - lo) / (hi - lo)
        hs = (np.arange(1 << 20, dtype=np.uint64) << 12)
        idx = np.linspace(0, (1 << 20) - 1, 4097).astype(np.int64)
        ups = 0
        for h in hs[idx]:
            v = O.scale_decode(E4M3, O.e4m3_code_sr(y, int(h)) & 0x7F)
            assert v in (lo, hi)
            ups += v == hi
        # sampled u on an even grid: the up-fraction is p to the sample's resolution
        assert abs(ups / idx.size - p) <= 1.0 / idx.size + 1e-12
        # the threshold itself: exactly the u >= 2^20 - floor(p * 2^20) round up,
        # so the up-count over all 2^20 variates is floor(p * 2^20)
        F = int(Fraction(y - lo) / Fraction(hi - lo) * 2 ** 20)
        T = 2 ** 20 - F
        if T <= 2 ** 20 - 1:
            assert O.scale_decode(E4M3, O.e4m3_code_sr(y, T << 12) & 0x7F) == hi
        if 1 <= T <= 2 ** 20:
            assert O.scale_decode(E4M3, O.e4m3_code_sr(y, ((T - 1) << 12) | 0xFFF) & 0x7F) == lo
    assert O.e4m3_code_sr(-2.25, 0xFFFFFFFF) == 0x80 | 0x41   # on grid: sign kept, unchanged
    assert O.e4m3_code_sr(449.0, 0xFFFFFFFF) == 0x7E          # saturates, never NaN


def test_requant_nan_blocks():
    """A NaN source block (NaN scale byte) makes x_hat NaN there: NVFP4
    column blocks holding it get the NaN scale code, MXFP8 blocks 0xFF, and
    their elements code 0; other blocks are unaffected."""
    codes, scales, src = _random_source(32, 64, 4)
    scales = scales.copy()
    scales[5, 2] = 0x7F                                  # rows 5, columns 32..47
    ct, st = O.requant_t(codes, scales, **src, target="nvfp4", dst_amax=src["amax"], seed=1)
    assert np.all(st[32:48, 0] == 0x7F) and np.all(ct[32:48, :8] == 0)
    assert np.all(st[:32, :] != 0x7F) and np.all(st[48:, :] != 0x7F) and np.all(st[32:48, 1] != 0x7F)
    el, sc = O.requant_t(codes, scales, **src, target="mxfp8", seed=1)
    assert np.all(sc[32:48, 0] == 0xFF) and np.all(el[32:48, :] == 0)
    assert np.all(sc[:32] != 0xFF) and np.all(sc[48:] != 0xFF)


def test_mxfp8_sr_index_and_scale():
    """Each MXFP8 element is the E4M3 stochastic rounding of x * 2^-e, e the
    block's E8M0 exponent, with the counter hash of its own index in the
    output orientation ((row0 + r) * cols + c): every element of a block draws
    its own variate."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((4, 64)) * 3.0).astype(np.float32)
    el, sc = O.mxfp8_quantize_sr(x, seed=99, row0=3)
    for r in range(4):
        for c in range(64):
            e = int(sc[r, c // 32]) - 127
            y = float(np.float32(x[r, c]) * np.float32(2.0 ** -e))
            assert el[r, c] == O.e4m3_code_sr(y, O.sr_hash(99, (3 + r) * 64 + c)), (r, c)


def test_mxfp8_non_finite_blocks():
    """A NaN or an infinity in a 32-element block has no power-of-two scale:
    the block's E8M0 byte is the NaN code 0xFF and its elements are 0; the
    other block of the row is unaffected."""
    x = np.ones((2, 64), np.float32)
    x[0, 5] = np.inf
    x[1, 40] = np.nan
    el, sc = O.mxfp8_quantize_sr(x, seed=1)
    assert sc[0, 0] == 0xFF and np.all(el[0, :32] == 0) and sc[0, 1] != 0xFF
    assert sc[1, 1] == 0xFF and np.all(el[1, 32:] == 0) and sc[1, 0] != 0xFF
    assert np.all(np.isnan(O.mxfp8_dequantize(el, sc)[0, :32]))


def test_dequantized_amax_is_the_max_of_the_dequantized_tensor():
    """The outer scale of a re-quantization is max |x_hat| over the whole
    dequantized tensor (the last row included), per-tensor or per-row source."""
    for per_row in (False, True):
        codes, scales, src = _random_source(32, 64, 5, per_row=per_row)
        scales, codes = scales.copy(), codes.copy()
        scales[31, 3] = 0x7E  # the largest block scale and code 6, in the last row's last block
        codes[31, 24:32] = 0x77
        if per_row:
            xh = np.concatenate([O.dequantize(codes[r:r + 1], scales[r:r + 1], float(src["row_amaxes"][r]))
                                 for r in range(32)])
        else:
            xh = O.dequantize(codes, scales, float(src["amax"]))
        want = np.max(np.abs(xh))
        if not per_row:  # the planted block holds the maximum
            assert np.argmax(np.abs(xh).max(axis=1)) == 31
        assert O.dequantized_amax(codes, scales, **src) == want


def test_requant_rejects_ragged_rows():
    codes, scales, src = _random_source(16, 32, 2)
    with pytest.raises(ValueError):
        O.requant_t(codes, scales, **src, target="mxfp8")        # 16 rows: not a multiple of 32
    O.requant_t(codes, scales, **src, target="nvfp4", dst_amax=1.0)


def test_strip_with_offset_is_the_full_result_rows():
    """A strip of source columns col0.. re-quantized with col0 gives exactly
    the rows col0.. of the whole tensor's result (both targets): the SR
    indices of a strip are those of the wider output."""
    rng = np.random.default_rng(11)
    rows, cols = 64, 48
    codes = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0x28, 0x50, (rows, cols // 16), dtype=np.uint8)
    for target, kw in (("mxfp8", {}), ("nvfp4", {"dst_amax": 9.0})):
        full = O.requant_t(codes, scales, amax=50.0, target=target, seed=5, **kw)
        for c0 in (0, 16, 32):
            part = O.requant_t(np.ascontiguousarray(codes[:, c0 // 2:c0 // 2 + 8]),
                               np.ascontiguousarray(scales[:, c0 // 16:c0 // 16 + 1]),
                               amax=50.0, target=target, seed=5, col0=c0, **kw)
            for f, p in zip(full, part):
                assert np.array_equal(f[c0:c0 + 16], p), (target, c0)
