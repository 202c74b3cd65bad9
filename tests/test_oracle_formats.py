"""Pins of the oracle's number formats against what the pages fix and against
independent library routines (numpy's ties-to-even rint, torch's OCP
float8_e4m3fn and bfloat16 casts).  CPU only."""
import numpy as np
import pytest
import torch

import oracle as O

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _f32(v):
    return np.float32(v)


def test_e2m1_grid_matches_pages(pages):
    mags = pages["e2m1_grid"]["magnitudes"]
    assert [O.e2m1_value(c) for c in range(8)] == mags
    assert [O.e2m1_value(8 | c) for c in range(8)] == [-m for m in mags]
    # every grid value (and its negative) encodes to itself
    for c, m in enumerate(mags):
        assert O.e2m1_code(m) == c
        assert O.e2m1_code(-m) == 8 | c


def test_e2m1_step_sizes(pages):
    mags = pages["e2m1_grid"]["magnitudes"]
    for lo, hi, step in pages["e2m1_steps"]["intervals"]:
        inside = [m for m in mags if lo <= m <= hi]
        assert np.allclose(np.diff(inside), step)


def test_five_goes_to_four_or_six(pages):
    ex = pages["five_is_forced"]
    v = O.e2m1_value(O.e2m1_code(ex["y"]))
    assert v in ex["allowed"]
    assert v == 4.0  # round-to-nearest-even: code 6 (value 4) is even


def _rne_by_binade(a):
    """Textbook ties-to-even rounding (numpy rint) at the local E2M1 step,
    saturated at 6: an independent statement of E2M1 RNE."""
    a = np.asarray(a, dtype=np.float64)
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    return np.minimum(np.rint(a / step) * step, 6.0)


def test_e2m1_rne_equals_rint_per_binade():
    rng = np.random.default_rng(7)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    near = np.concatenate([np.nextafter(mids, np.float32(0)), mids,
                           np.nextafter(mids, np.float32(10))])
    rand = rng.uniform(0, 9, 20000).astype(np.float32)
    tiny = np.array([0.0, 1e-45, 1e-38, 1e-20, 0.1, 6.0, 7.0, 8.0, 1e30], np.float32)
    ys = np.concatenate([near, rand, tiny])
    ref = _rne_by_binade(ys)
    got = np.array([O.e2m1_value(O.e2m1_code(float(y))) for y in ys])
    assert np.array_equal(got, ref)
    gotn = np.array([O.e2m1_value(O.e2m1_code(-float(y))) for y in ys])
    assert np.array_equal(gotn, -ref)


def test_e2m1_sign_of_zero():
    assert O.e2m1_code(0.0) == 0
    assert O.e2m1_code(-0.0) == 8
    assert O.e2m1_code(-0.1) == 8
    assert O.e2m1_code(-1e-40) == 8


def test_e4m3_decode_matches_torch_for_all_bytes():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        got = O.scale_decode("e4m3", c)
        if np.isnan(ref[c]):
            assert np.isnan(got), c
        else:
            assert got == ref[c], (c, got, ref[c])


def test_e4m3_range_and_nvfp4_range(pages):
    r = pages["nvfp4_range"]
    assert O.scale_decode("e4m3", 0x7E) == 448.0
    assert np.isnan(O.scale_decode("e4m3", 0x7F))
    smallest_e4m3 = O.scale_decode("e4m3", 0x01)
    assert 0.5 * smallest_e4m3 == r["min"]
    assert 6.0 * O.scale_decode("e4m3", 0x7E) == r["max"]
    assert 2 * 0.5 * smallest_e4m3 == r["alpha2_min"]
    assert 2 * 6.0 * 448.0 == r["alpha2_max"]


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(11)
    codes = np.arange(0x7F)
    vals = np.array([O.scale_decode("e4m3", c) for c in codes])
    mids = (vals[:-1] + vals[1:]) / 2
    cand = np.concatenate([vals, mids, rng.uniform(0, 448, 20000),
                           np.exp(rng.uniform(np.log(1e-4), np.log(448), 20000))]).astype(np.float32)
    cand = np.concatenate([cand, np.nextafter(cand, np.float32(0)), np.nextafter(cand, np.float32(1e9))])
    cand = cand[(cand >= 0) & (cand <= 448)]
    ref = torch.from_numpy(cand).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([O.scale_encode("e4m3", float(v)) for v in cand], np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(cand[i]), int(got[i]), int(ref[i])) for i in bad[:10]]


def test_e4m3_encode_saturates_above_max():
    for v in [448.0, 449.0, 463.9, 464.0, 480.0, 1e6, 3.0e38, float("inf")]:
        assert O.scale_encode("e4m3", v) == 0x7E


def _minifloat_fn(code, ebits, mbits, signed):
    """Decode one byte of an FN-style minifloat (no infinities; the all-ones
    pattern is NaN; exponent field 0 holds the subnormals) with the bias
    2^(ebits-1) - 1 that the "UE5M3" blog's emulation uses (实现).  Written
    here independently of the oracle; for ebits=4, mbits=3, signed it is the
    OCP E4M3FN byte (checked against torch below)."""
    bias = 2 ** (ebits - 1) - 1
    sign = -1.0 if (signed and code >> (ebits + mbits) & 1) else 1.0
    body = code & ((1 << (ebits + mbits)) - 1)
    if body == (1 << (ebits + mbits)) - 1:
        return float("nan")
    e, m = body >> mbits, body & ((1 << mbits) - 1)
    if e == 0:
        return sign * m / 2 ** mbits * 2.0 ** (1 - bias)
    return sign * (1 + m / 2 ** mbits) * 2.0 ** (e - bias)


def test_minifloat_construction_reproduces_torch_e4m3fn():
    # the construction the UE5M3 pins rest on, checked on the one format a
    # library defines: every E4M3FN byte
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    got = np.array([_minifloat_fn(c, 4, 3, True) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok].astype(np.float64))


def test_ue5m3_is_unsigned_5_exponent_3_mantissa_bits():
    """"UE5M3" blog (数学推导; 背景): the block scale is unsigned with 5
    exponent and 3 mantissa bits.  The oracle's decode equals the same
    construction with ebits=5, mbits=3 and no sign bit for every byte: bit 7
    is an exponent bit (0x80 decodes to +2, not to -0), every binade holds 8
    codes spaced by a 1/8 of its base, and the bias is 2^4 - 1 = 15."""
    for c in range(256):
        want = _minifloat_fn(c, 5, 3, False)
        got = O.scale_decode("ue5m3", c)
        if np.isnan(want):
            assert np.isnan(got), c
        else:
            assert got == want, (c, got, want)
    assert O.scale_decode("ue5m3", 0x80) == 2.0
    vals = [O.scale_decode("ue5m3", c) for c in range(255)]
    assert all(v >= 0 for v in vals)
    assert all(b > a for a, b in zip(vals, vals[1:]))  # unsigned: code order = value order
    for e in range(1, 31):  # 8 codes per binade, spaced base / 8
        base = 2.0 ** (e - 15)
        assert [vals[8 * e + m] for m in range(8)] == [base + m * base / 8 for m in range(8)]
    # the top binade is 2^(2^5 - 1 - 15) = 2^16, the emulation's exponent ceiling
    assert vals[0xF8] == 2.0 ** 16


def test_ue5m3_rounding_matches_the_pages_mantissa_rule():
    """The "UE5M3" blog's emulation (实现) rounds a positive scale within its
    binade 2^e (e = floor(log2 s), clamped to [-bias, 2^5 - 1 - bias]) to 3
    fractional mantissa bits, ties to even.  Over the normal range of the
    format (2^-14 .. 114688) the oracle's encoder gives exactly that value;
    below 2^-14 the format reading adds subnormals (step 2^-17) and at the top
    it saturates at 0xFE, where the emulation is not a format (it carries past
    the exponent field)."""
    rng = np.random.default_rng(11)
    s = np.concatenate([2.0 ** rng.uniform(-14, np.log2(114688.0), 4000),
                        [2.0 ** -14, 1.0, 1.0625, 1.1875, 3.0, 448.0, 1000.0, 114688.0]])
    s = s.astype(np.float32).astype(np.float64)
    # exact ties (half way between two codes) and their neighbours
    mids = np.array([(1 + (m + 0.5) / 8) * 2.0 ** e for e in (-10, 0, 7, 15) for m in range(7)])
    s = np.concatenate([s, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9)]).astype(np.float32)
    for v in s.astype(np.float64):
        e = int(np.floor(np.log2(v)))
        e = min(max(e, -15), 2 ** 5 - 1 - 15)
        want = np.rint(v / 2.0 ** e * 8) / 8 * 2.0 ** e
        if want > 114688.0:
            want = 114688.0
        got = O.scale_decode("ue5m3", O.scale_encode("ue5m3", float(v)))
        assert got == want, (float(v), got, want)


def test_ue5m3_range_is_wider_than_e4m3():
    """"UE5M3" blog (直觉解释): one more exponent bit doubles the range the
    scale can span, at the same 3 mantissa bits.  Against the torch-pinned
    E4M3 byte: the largest value grows by 2^8 and the smallest by 2^-8, the
    log2 span roughly doubles, and where both formats have normal binades
    (2^-6 .. 448) they hold exactly the same values."""
    ue = np.array([O.scale_decode("ue5m3", c) for c in range(255)])
    e4 = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert ue.max() == 256 * e4.max()
    assert ue[ue > 0].min() == e4[e4 > 0].min() / 256
    span_ue = np.log2(ue.max() / ue[ue > 0].min())
    span_e4 = np.log2(e4.max() / e4[e4 > 0].min())
    assert 1.8 < span_ue / span_e4 < 2.2
    lo, hi = 2.0 ** -6, 448.0
    assert np.array_equal(ue[(ue >= lo) & (ue <= hi)], e4[(e4 >= lo) & (e4 <= hi)])


def test_ue5m3_encode_closed_form():
    # the format's own ends: subnormal step 2^-17, largest 0xFE, NaN 0xFF,
    # saturation, and encode(decode(c)) = c
    vals = [O.scale_decode("ue5m3", c) for c in range(255)]
    assert vals[1] == 2.0 ** -17 and vals[8] == 2.0 ** -14
    assert vals[0xFE] == 114688.0 == 1.75 * 2 ** 16
    assert np.isnan(O.scale_decode("ue5m3", 0xFF))
    assert O.scale_encode("ue5m3", 1e9) == 0xFE
    for c in range(255):
        assert O.scale_encode("ue5m3", vals[c]) == c


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(3)
    f = np.concatenate([rng.standard_normal(5000) * 100, rng.standard_normal(5000) * 1e-39,
                        [0.0, -0.0, 1.0, 3.0e38, -3.4e38, 1.00390625, 1.01171875]]).astype(np.float32)
    # exact ties: low 16 bits = 0x8000
    u = f.view(np.uint32)
    ties = ((u & 0xFFFF0000) | 0x8000).view(np.float32)
    f = np.concatenate([f, ties])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([O.f32_to_bf16(float(v)) for v in f], np.uint16)
    assert np.array_equal(got, ref)


def test_fmix32_published_vectors(pages):
    v = pages["murmur3_vectors"]
    assert O.fmix32(1) == int(v["seed1"], 16)
    assert O.fmix32(0xFFFFFFFF) == int(v["seedFFFFFFFF"], 16)
    assert O.fmix32(0) == int(v["seed0"], 16)


def test_sr_hash_key_construction():
    """The counter hash is fmix32 (pinned above to MurmurHash3's published
    finalizer) applied to lo32(idx) ^ k, with the key
    k = fmix32(lo32(seed) ^ fmix32(hi32(seed) ^ hi32(idx) ^ C)) and C the
    32-bit golden-ratio constant floor(2^32 / phi).  The pages leave the
    random source of stochastic rounding open; this pins the constant to its
    published definition and each word of seed and index to its place."""
    phi = (1 + 5 ** 0.5) / 2
    C = int(2 ** 32 / phi)
    assert C == 0x9E3779B9
    M = 0xFFFFFFFF
    for seed in (0, 1234, 0xDEADBEEF12345678, (7 << 32) | 3):
        for idx in (0, 1, 15, 123456789, (1 << 32) + 5, (0xABCDE << 32) | 0x1234):
            k = O.fmix32((seed & M) ^ O.fmix32((seed >> 32) ^ (idx >> 32) ^ C))
            assert O.sr_hash(seed, idx) == O.fmix32((idx & M) ^ k), (seed, idx)


def test_sr_hash_uniformity():
    n = 1 << 16
    u = np.array([O.sr_hash(1234, i) >> 8 for i in range(n)], np.float64) / 2 ** 24
    hist, _ = np.histogram(u, bins=64, range=(0, 1))
    exp = n / 64
    chi2 = ((hist - exp) ** 2 / exp).sum()
    assert chi2 < 120  # 63 dof; p ~ 1e-5
    assert abs(u.mean() - 0.5) < 5 * np.sqrt(1 / 12 / n)
    # the high word of the index and of the seed both reach the hash
    assert O.sr_hash(1234, 5) != O.sr_hash(1234, 5 + (1 << 32))
    assert O.sr_hash(1234, 5) != O.sr_hash(1234 + (1 << 32), 5)
