"""GPU-vs-oracle parity, through the C ABI, of the re-quantization for the
backward pass ("End-to-End 4-Bit Training", Re-quantization with stochastic
rounding): dequantize -> transpose -> stochastic re-quantization to NVFP4 or
MXFP8, the dequantized amax, and the E4M3 stochastic-rounding element
encoder.  Sources are quantized by the oracle (seeded synthetic tensors).

Bar: every output byte bit-exact; the dequantized amax bit-exact."""
import numpy as np
import pytest

import oracle as O
from helpers import log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
nv = pytest.importorskip("nvfp4_block_scaled_02_amd")
from nvfp4_block_scaled_02_amd import _native as N  # noqa: E402
from nvfp4_block_scaled_02_amd import synth  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _same(got, ref, what):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{what}: differ at {len(bad)} positions, first {bad[:4].tolist()}"


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _source(rows, cols, seed, *, per_row=False, fmt="e4m3", select="4over6", spread=1.5):
    """An NVFP4 tensor quantized by the oracle from a seeded tensor."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)) * np.exp(rng.normal(0, spread, (rows, 1)))
    x[rng.random((rows, cols)) < 0.002] *= 40
    xb = synth.to_bf16_bits(x.astype(np.float32))
    f = O.FMT_E4M3 if fmt == "e4m3" else O.FMT_UE5M3
    sel = O.SELECT_4OVER6 if select == "4over6" else O.SELECT_6
    gmax = O.default_global_max(f, sel)
    if per_row:
        ra = O.row_amax(xb)
        c, s, _ = O.quantize_rowscaled(xb, ra, fmt=f, select=sel)
        return dict(codes=c, scales=s, row_amaxes=ra, amax=None, gmax=gmax, fmt=fmt, f=f)
    A = O.tensor_amax(xb)
    c, s, _ = O.quantize(xb, A, fmt=f, select=sel)
    return dict(codes=c, scales=s, row_amaxes=None, amax=np.float32(A), gmax=gmax, fmt=fmt, f=f)


def _gpu_src(src):
    kw = dict(global_max=src["gmax"], fmt=src["fmt"])
    if src["row_amaxes"] is not None:
        kw["row_amaxes"] = _dev(src["row_amaxes"])
    else:
        kw["amax"] = _dev(np.array([src["amax"]], np.float32))
    return _dev(src["codes"]), _dev(src["scales"]), kw


def _oracle_src(src):
    kw = dict(fmt=src["f"], global_max=src["gmax"])
    if src["row_amaxes"] is not None:
        kw["row_amaxes"] = src["row_amaxes"]
    else:
        kw["amax"] = float(src["amax"])
    return kw


def _run(src, target, seed, dst_amax=None, dst_fmt="e4m3"):
    c, s, kw = _gpu_src(src)
    dk = {}
    if target == "nvfp4":
        dk = dict(dst_amax=_dev(np.array([dst_amax], np.float32)), dst_fmt=dst_fmt)
    ot, st = nv.requantize_t(c, s, target=target, seed=seed, **kw, **dk)
    torch.cuda.synchronize()
    return ot.cpu().numpy(), st.cpu().numpy()


def _ref(src, target, seed, dst_amax=None, dst_fmt="e4m3"):
    kw = _oracle_src(src)
    dk = {}
    if target == "nvfp4":
        dk = dict(dst_amax=dst_amax, dst_fmt=O.FMT_E4M3 if dst_fmt == "e4m3" else O.FMT_UE5M3)
    return O.requant_t(src["codes"], src["scales"], target=target, seed=seed, **kw, **dk)


# ---------------------------------------------------------------- encoder
def test_e4m3_sr_encoder_matches_oracle():
    """Clamp + E4M3 stochastic rounding of single values, every byte position,
    against the oracle's rule: random values over every binade (subnormals,
    above 448, negatives, zeros) with random variates, and variates placed on
    both sides of each value's 20-bit threshold."""
    rng = np.random.default_rng(42)
    ys = [np.ldexp(1.0 + rng.random(400), e) for e in range(-14, 9)]
    ys.append(448.0 + 100.0 * rng.random(200))
    ys.append(np.array([0.0, -0.0, 448.0, -448.0, 2.25, -2.25, 1e-30, -1e-30, 3e38, -3e38]))
    y = np.concatenate(ys).astype(np.float32)
    y = np.concatenate([y, -y[::3]])
    h = rng.integers(0, 2 ** 32, size=y.size, dtype=np.uint64).astype(np.uint32)
    # thresholds: the smallest variate that rounds up (per the 20-bit rule) and one below
    grid = np.array([O.scale_decode(O.FMT_E4M3, c) for c in range(0x7F)])
    ty, th = [], []
    for v in np.abs(y[:3000:7]).astype(np.float64):
        if v >= 448.0:
            continue
        j = np.searchsorted(grid, v, side="right") - 1
        p = (v - grid[j]) / (grid[j + 1] - grid[j])
        F = int(np.floor(p * 2 ** 20))
        if F == 0:
            continue
        thr = (2 ** 20 - F) << 12
        for hv in (thr, thr - 1, min(thr + 4095, 2 ** 32 - 1)):
            ty.append(v)
            th.append(hv)
    y = np.concatenate([y, np.array(ty, np.float32)])
    h = np.concatenate([h, np.array(th, np.uint64).astype(np.uint32)])
    n = y.size - y.size % 4
    y, h = y[:n], h[:n]
    out = torch.empty(n, dtype=torch.uint8, device="cuda")
    dy, dh = _dev(y), _dev(h)  # held until the kernel has run (no allocator reuse)
    N.check(N.lib().nvfp4_test_e4m3_sr(dy.data_ptr(), dh.data_ptr(), n, out.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream), "test_e4m3_sr")
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = np.array([O.e4m3_code_sr(float(a), int(b)) for a, b in zip(y, h)], np.uint8)
    _same(got, ref, "E4M3 SR bytes")


# ---------------------------------------------------------------- dequantized amax
@pytest.mark.parametrize("rows,cols,per_row,fmt", [
    (64, 144, False, "e4m3"), (37, 48, True, "e4m3"), (512, 1024, False, "ue5m3"),
    (1, 16, False, "e4m3"), (300, 4112, True, "e4m3"),
])
def test_dequantized_amax(rows, cols, per_row, fmt):
    log(f"dequantized_amax {rows}x{cols} per_row={per_row} {fmt}")
    src = _source(rows, cols, rows * 7 + cols, per_row=per_row, fmt=fmt,
                  select="6" if fmt == "ue5m3" else "4over6")
    c, s, kw = _gpu_src(src)
    got = nv.dequantized_amax(c, s, **kw).cpu().numpy()
    ref = np.float32(O.dequantized_amax(src["codes"], src["scales"], **_oracle_src(src)))
    _same(got.view(np.uint32), np.array([ref]).view(np.uint32), "dequantized amax")


def test_dequantized_amax_nan():
    src = _source(32, 64, 3)
    src["scales"] = src["scales"].copy()
    src["scales"][4, 1] = 0x7F
    c, s, kw = _gpu_src(src)
    assert np.isnan(nv.dequantized_amax(c, s, **kw).cpu().numpy()[0])
    assert np.isnan(O.dequantized_amax(src["codes"], src["scales"], **_oracle_src(src)))


# ---------------------------------------------------------------- re-quantization
SHAPES = [(32, 16), (64, 144), (96, 400), (160, 128), (320, 272), (2112, 48), (64, 4096)]


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("per_row", [False, True])
def test_requant_mxfp8(rows, cols, per_row):
    log(f"requant mxfp8 {rows}x{cols} per_row={per_row}")
    src = _source(rows, cols, rows + 3 * cols, per_row=per_row)
    got = _run(src, "mxfp8", seed=1234)
    ref = _ref(src, "mxfp8", seed=1234)
    _same(got[1], ref[1], f"mxfp8 scales {rows}x{cols}")
    _same(got[0], ref[0], f"mxfp8 elements {rows}x{cols}")


@pytest.mark.parametrize("rows,cols", SHAPES + [(48, 48), (16, 272), (80, 16)])
@pytest.mark.parametrize("per_row", [False, True])
def test_requant_nvfp4(rows, cols, per_row):
    log(f"requant nvfp4 {rows}x{cols} per_row={per_row}")
    src = _source(rows, cols, rows + 5 * cols, per_row=per_row)
    A2 = O.dequantized_amax(src["codes"], src["scales"], **_oracle_src(src))
    got = _run(src, "nvfp4", seed=77, dst_amax=A2)
    ref = _ref(src, "nvfp4", seed=77, dst_amax=A2)
    _same(got[1], ref[1], f"nvfp4 scales_t {rows}x{cols}")
    _same(got[0], ref[0], f"nvfp4 codes_t {rows}x{cols}")


@pytest.mark.parametrize("src_fmt,dst_fmt", [("ue5m3", "e4m3"), ("e4m3", "ue5m3"), ("ue5m3", "ue5m3")])
def test_requant_formats(src_fmt, dst_fmt):
    log(f"requant formats {src_fmt} -> {dst_fmt}")
    src = _source(96, 272, 9, fmt=src_fmt, select="6" if src_fmt == "ue5m3" else "4over6")
    A2 = O.dequantized_amax(src["codes"], src["scales"], **_oracle_src(src))
    got = _run(src, "nvfp4", seed=5, dst_amax=A2, dst_fmt=dst_fmt)
    ref = _ref(src, "nvfp4", seed=5, dst_amax=A2, dst_fmt=dst_fmt)
    _same(got[1], ref[1], "scales_t")
    _same(got[0], ref[0], "codes_t")
    got = _run(src, "mxfp8", seed=5)
    ref = _ref(src, "mxfp8", seed=5)
    _same(got[1], ref[1], "mxfp8 scales")
    _same(got[0], ref[0], "mxfp8 elements")


def test_requant_special_blocks():
    """NaN scale bytes in the source, a NaN and a negative row amax, a zero
    row, and a stale outer amax below the dequantized one (saturation)."""
    src = _source(64, 160, 21, per_row=True)
    src["scales"] = src["scales"].copy()
    src["scales"][3, 2] = 0x7F
    src["row_amaxes"] = src["row_amaxes"].copy()
    src["row_amaxes"][10] = np.nan
    src["row_amaxes"][11] = -1.0
    src["row_amaxes"][12] = 0.0
    src["codes"] = src["codes"].copy()
    src["codes"][13, :] = 0
    A2 = O.dequantized_amax(src["codes"], src["scales"], **_oracle_src(src))
    assert np.isnan(A2)
    for dst in (float(np.nanmax(np.abs(O.dequantize_rowscaled(src["codes"], src["scales"],
                                                                src["row_amaxes"])))) * 0.5,
                float("nan"), 0.0):
        got = _run(src, "nvfp4", seed=3, dst_amax=dst)
        ref = _ref(src, "nvfp4", seed=3, dst_amax=dst)
        _same(got[1], ref[1], f"scales_t dst {dst}")
        _same(got[0], ref[0], f"codes_t dst {dst}")
    got = _run(src, "mxfp8", seed=3)
    ref = _ref(src, "mxfp8", seed=3)
    _same(got[1], ref[1], "mxfp8 scales specials")
    _same(got[0], ref[0], "mxfp8 elements specials")


def test_requant_deterministic_and_seeded():
    src = _source(128, 256, 4)
    a = _run(src, "mxfp8", seed=11)
    b = _run(src, "mxfp8", seed=11)
    c = _run(src, "mxfp8", seed=12)
    _same(a[0], b[0], "same seed")
    assert (a[0] != c[0]).mean() > 0.05


# ---------------------------------------------------------------- full size
@pytest.mark.parametrize("target", ["mxfp8", "nvfp4"])
def test_requant_full_activation_per_token(target):
    """The saved activation of the pages' linear layer: 8192x4096, per-token
    outer scales, Four-Over-Six; re-quantized transposed for the backward."""
    log(f"requant full activation per-token -> {target}")
    xb = synth.make("activation")["x"]
    ra = O.row_amax(xb)
    c, s, _ = O.quantize_rowscaled(xb, ra, select=O.SELECT_4OVER6)
    src = dict(codes=c, scales=s, row_amaxes=ra, amax=None, gmax=256.0, fmt="e4m3", f=O.FMT_E4M3)
    A2 = O.dequantized_amax(c, s, **_oracle_src(src)) if target == "nvfp4" else None
    got = _run(src, target, seed=1234, dst_amax=A2)
    ref = _ref(src, target, seed=1234, dst_amax=A2)
    _same(got[1], ref[1], f"{target} scales full")
    _same(got[0], ref[0], f"{target} elements full")


def test_requant_full_weight_per_tensor():
    """A 14336x4096 weight quantized per tensor (max->6, S_g = 448), to MXFP8."""
    log("requant full weight 14336x4096 -> mxfp8")
    xb = synth.make("qat")["x"]
    A = O.tensor_amax(xb)
    c, s, _ = O.quantize(xb, A, select=O.SELECT_6, global_max=448.0)
    src = dict(codes=c, scales=s, row_amaxes=None, amax=np.float32(A), gmax=448.0, fmt="e4m3",
               f=O.FMT_E4M3)
    got = _run(src, "mxfp8", seed=99)
    ref = _ref(src, "mxfp8", seed=99)
    _same(got[1], ref[1], "weight mxfp8 scales")
    _same(got[0], ref[0], "weight mxfp8 elements")
