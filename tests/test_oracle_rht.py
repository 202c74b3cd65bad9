"""Pins of the oracle's 16-point random Hadamard transform and its use before
NVFP4 quantization ("Four Over Six" notes, Method: NVIDIA's recipe applies an
RHT to both inputs of the weight-gradient GEMM; "End-to-End 4-Bit
Training", Quantized communications: an orthogonal rotation that spreads
outliers, inverted exactly).  Checked against scipy's Sylvester Hadamard
matrix, orthogonality, the outlier-spreading and smaller-scale claims, and
the composition with the already pinned quantizer.  CPU only."""
import numpy as np
import pytest
from scipy.linalg import hadamard

import oracle as O

H16 = hadamard(16).astype(np.float64)


def _signs(seed):
    m = O.rht_signs(seed)
    return np.array([-1.0 if (m >> j) & 1 else 1.0 for j in range(16)])


def _bf16(x):
    u = np.asarray(x, np.float32).view(np.uint32)
    return (((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16).view(np.float32)


def test_transform_is_the_sylvester_hadamard_product():
    """Exact on dyadic inputs (every binary32 step exact); within rounding on
    random bf16 data, against H16 diag(s) x / 4 in binary64."""
    rng = np.random.default_rng(0)
    for seed in (0, 1, 77):
        s = _signs(seed)
        x = rng.integers(-64, 64, 16).astype(np.float32) * np.float32(0.5)
        assert np.array_equal(O.rht16(x, seed), (H16 @ (s * x)) / 4)
        for _ in range(50):
            x = _bf16(rng.standard_normal(16) * 10.0 ** rng.uniform(-3, 3))
            ref = (H16 @ (s * x.astype(np.float64))) / 4
            assert np.all(np.abs(O.rht16(x, seed) - ref) <= 8 * 2.0 ** -24 * np.abs(x).sum() / 4 + 1e-45)


def test_inverse_and_energy():
    rng = np.random.default_rng(1)
    for seed in (3, 4):
        x = rng.integers(-1000, 1000, 16).astype(np.float32)
        assert np.array_equal(O.rht16(O.rht16(x, seed), seed, inverse=True), x)  # exact inputs
        for _ in range(50):
            x = _bf16(rng.standard_normal(16))
            y = O.rht16(x, seed)
            assert abs(float((y.astype(np.float64) ** 2).sum() / (x.astype(np.float64) ** 2).sum()) - 1) < 1e-6
            back = O.rht16(y, seed, inverse=True)
            assert np.all(np.abs(back - x) <= 1e-6 * np.abs(x).max())


def test_single_outlier_is_spread_evenly():
    """A block holding one nonzero value v becomes 16 values of magnitude
    |v| / 4: the outlier is spread over the block ([E2E] figure)."""
    for j in (0, 5, 15):
        x = np.zeros(16, np.float32)
        x[j] = -500.0
        y = O.rht16(x, 9)
        assert np.all(np.abs(y) == 125.0)


def test_sign_vector_is_seeded():
    # s_j = -1 iff the top bit of the counter hash (pinned in the formats
    # tests) of index j under the sign seed is set
    for seed in (0, 7, 1234, (5 << 32) | 9):
        want = sum(1 << j for j in range(16) if O.sr_hash(seed, j) >> 31)
        assert O.rht_signs(seed) == want
    m = [O.rht_signs(s) for s in range(200)]
    assert len(set(m)) > 190 and O.rht_signs(7) == O.rht_signs(7)
    neg = np.mean([bin(v).count("1") for v in m]) / 16
    assert 0.4 < neg < 0.6


def _outlier_tensor(rows, cols, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols))
    x[rng.random((rows, cols)) < 0.01] *= 40  # sparse outliers
    return _bf16(x.astype(np.float32))


@pytest.mark.parametrize("axis", [O.AXIS_ROW, O.AXIS_COL])
def test_quantize_rht_is_quantize_of_the_transformed_tensor(axis):
    x = _outlier_tensor(64, 96, 2)
    s = _signs(11)
    if axis == O.AXIS_ROW:
        t = ((H16 @ (s[:, None] * x.reshape(-1, 16).T.astype(np.float64))) / 4).T.reshape(x.shape)
    else:
        xt = x.T.reshape(-1, 16).T.astype(np.float64)            # column blocks as columns
        t = ((H16 @ (s[:, None] * xt)) / 4).T.reshape(x.shape[1], x.shape[0]).T
    t32 = np.empty_like(x)
    # the transform in the oracle's own binary32 order, for the exact comparison
    if axis == O.AXIS_ROW:
        for i in range(x.shape[0]):
            for c in range(0, x.shape[1], 16):
                t32[i, c:c + 16] = O.rht16(x[i, c:c + 16], 11)
    else:
        for r in range(0, x.shape[0], 16):
            for c in range(x.shape[1]):
                t32[r:r + 16, c] = O.rht16(x[r:r + 16, c], 11)
    assert np.all(np.abs(t32 - t) <= 1e-5 * np.abs(t).max())
    A = O.rht_amax(x, axis=axis, sign_seed=11)
    assert A == np.abs(t32).max()
    for rnd in (O.ROUND_RNE, O.ROUND_SR):
        sel = O.SELECT_6 if rnd == O.ROUND_SR else O.SELECT_4OVER6
        got = O.quantize_rht(x, A, axis=axis, sign_seed=11, select=sel, rounding=rnd, seed=5)
        ref = (O.quantize(t32, A, select=sel, rounding=rnd, seed=5) if axis == O.AXIS_ROW
               else O.quantize_cols(t32, A, select=sel, rounding=rnd, seed=5))
        for g, r in zip(got, ref):
            assert np.array_equal(g, r)


def test_rht_lets_outlier_blocks_take_a_smaller_scale():
    """The transform smooths a block with an outlier so that it is quantized
    with a smaller scale factor ([E2E] Quantized communications): for blocks
    whose largest value is an outlier v, the transformed block's maximum is
    at most (|v| + sum of the others) / 4, and its max->6 scale code is
    smaller than the untransformed one (same outer scale)."""
    rng = np.random.default_rng(3)
    x = _bf16(rng.standard_normal((64, 16)).astype(np.float32))
    x[np.arange(64), rng.integers(0, 16, 64)] = _bf16(np.float32(60.0) * rng.choice([-1, 1], 64))
    A = np.float32(60.0)
    c, s, _ = O.quantize(x, A, select=O.SELECT_6, global_max=448.0)
    cr, sr, _ = O.quantize_rht(x, A, sign_seed=1, select=O.SELECT_6, global_max=448.0)
    y = np.stack([O.rht16(b, 1) for b in x])
    bound = (np.abs(x).sum(axis=1)) / 4
    assert np.all(np.abs(y).max(axis=1) <= bound * (1 + 1e-6))
    assert np.all(sr[:, 0] < s[:, 0])


def test_dequantize_rht_inverts_exact_values():
    """Values exactly representable after the transform come back exactly:
    build y on the grid, x = RHT^-1(y) exact (dyadic), then quantize_rht(x)
    recovers y and dequantize_rht returns x."""
    rng = np.random.default_rng(4)
    q = rng.choice([0, 0.5, 1, 1.5, 2, 3, 4, 6], size=(4, 64)) * rng.choice([-1, 1], size=(4, 64))
    q[:, ::16] = 6.0
    y = (q * 4.0).astype(np.float32)  # scale code 4 (0x48) with alpha = 1
    x = np.concatenate([O.rht16(b, 21, inverse=True) for b in y.reshape(-1, 16)]).reshape(y.shape)
    assert np.array_equal(np.concatenate([O.rht16(b, 21) for b in x.reshape(-1, 16)]).reshape(y.shape), y)
    A = np.float32(6 * 448)
    c, s, _ = O.quantize_rht(x, A, sign_seed=21, select=O.SELECT_6, global_max=448.0)
    assert np.all(s == 0x48)
    assert np.array_equal(O.dequantize_rht(c, s, A, sign_seed=21, global_max=448.0), x)


@pytest.mark.parametrize("axis", [O.AXIS_ROW, O.AXIS_COL])
def test_strip_with_offset_is_the_full_result_rows(axis):
    """Row or column strips quantized with out_row0 reproduce the rows
    out_row0.. of the whole tensor's output (SR indices of the wider output)."""
    x = _outlier_tensor(48, 64, 7)
    A = O.rht_amax(x, axis=axis, sign_seed=3)
    kw = dict(axis=axis, sign_seed=3, select=O.SELECT_6, rounding=O.ROUND_SR, seed=99)
    full = O.quantize_rht(x, A, **kw)
    for o in (0, 16, 32):
        strip = x[o:o + 16] if axis == O.AXIS_ROW else x[:, o:o + 16]
        part = O.quantize_rht(np.ascontiguousarray(strip), A, out_row0=o, **kw)
        for f, p in zip(full[:2], part[:2]):
            assert np.array_equal(f[o:o + 16], p), o
