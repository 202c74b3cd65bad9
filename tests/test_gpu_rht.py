"""GPU-vs-oracle parity, through the C ABI, of the 16-point random Hadamard
transform around NVFP4 quantization ("Four Over Six" notes, Method; "End-to-
End 4-Bit Training", Quantized communications): the transformed tensor's
amax, quantization of row blocks and of column blocks (the weight-gradient
operands), and dequantization followed by the inverse transform.

Bar: amax, codes, scale bytes and counts bit-exact; binary32 outputs
bit-exact (the same operation order on both sides)."""
import numpy as np
import pytest

import oracle as O
from helpers import dev_bf16, dev_f32, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
nv = pytest.importorskip("nvfp4_block_scaled_02_amd")
from nvfp4_block_scaled_02_amd import synth  # noqa: E402

AX = {"row": O.AXIS_ROW, "col": O.AXIS_COL}


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _same(got, ref, what):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{what}: differ at {len(bad)} positions, first {bad[:4].tolist()}"


def _tensor(rows, cols, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)) * np.exp(rng.normal(0, 1.0, (rows, 1)))
    x[rng.random((rows, cols)) < 0.01] *= 40
    return synth.to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("rows,cols", [(16, 16), (48, 80), (160, 272), (1024, 1040)])
def test_rht_amax(axis, rows, cols):
    log(f"rht_amax {axis} {rows}x{cols}")
    xb = _tensor(rows, cols, rows + cols)
    got = nv.rht_amax(dev_bf16(xb), axis=axis, sign_seed=7).cpu().numpy()
    ref = np.float32(O.rht_amax(xb, axis=AX[axis], sign_seed=7))
    _same(got.view(np.uint32), np.array([ref]).view(np.uint32), "rht amax")


def test_rht_amax_nan():
    xb = _tensor(32, 64, 1)
    xf = O.as_f32(xb).copy()
    xf[20, 7] = np.nan
    xb = synth.to_bf16_bits(xf)
    for axis in ("row", "col"):
        assert np.isnan(nv.rht_amax(dev_bf16(xb), axis=axis).cpu().numpy()[0])


CASES = [("4over6", "rne", "e4m3"), ("6", "rne", "e4m3"), ("6", "sr", "ue5m3"),
         ("4over6-mae", "rne", "e4m3")]
SEL = {"6": O.SELECT_6, "4over6": O.SELECT_4OVER6, "4over6-mae": O.SELECT_4OVER6_MAE}


@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("select,rounding,fmt", CASES)
@pytest.mark.parametrize("rows,cols", [(16, 16), (48, 208), (160, 272), (512, 1024)])
def test_quantize_rht(axis, select, rounding, fmt, rows, cols):
    log(f"quantize_rht {axis} {select} {rounding} {fmt} {rows}x{cols}")
    xb = _tensor(rows, cols, 3 * rows + cols)
    A = np.float32(O.rht_amax(xb, axis=AX[axis], sign_seed=11))
    q = nv.quantize_rht(dev_bf16(xb), dev_f32(np.array([A], np.float32)), axis=axis, sign_seed=11,
                        fmt=fmt, select=select, rounding=rounding, seed=1234, count4=True)
    torch.cuda.synchronize()
    rc, rs, rn = O.quantize_rht(xb, A, axis=AX[axis], sign_seed=11, fmt=fmt, select=SEL[select],
                                rounding=O.ROUND_SR if rounding == "sr" else O.ROUND_RNE, seed=1234)
    _same(q.scales.cpu().numpy(), rs, "scales")
    _same(q.codes.cpu().numpy(), rc, "codes")
    assert int(q.count4.item()) == rn


@pytest.mark.parametrize("rows,cols", [(16, 16), (64, 272), (1024, 4096)])
def test_dequantize_rht(rows, cols):
    log(f"dequantize_rht {rows}x{cols}")
    xb = _tensor(rows, cols, rows)
    A = np.float32(O.rht_amax(xb, sign_seed=3))
    c, s, _ = O.quantize_rht(xb, A, sign_seed=3)
    gm = O.default_global_max(O.FMT_E4M3, O.SELECT_4OVER6)
    got = nv.dequantize_rht(torch.from_numpy(c).cuda(), torch.from_numpy(s).cuda(),
                            dev_f32(np.array([A], np.float32)), global_max=gm, sign_seed=3)
    torch.cuda.synchronize()
    ref = O.dequantize_rht(c, s, A, sign_seed=3)
    _same(got.cpu().numpy().view(np.uint32), ref.view(np.uint32), "x_hat after inverse")


def test_full_activation_col_rht():
    """The weight-gradient operand: the 8192x4096 activation quantized
    column-wise (blocks along tokens) after the transform, Four-Over-Six."""
    log("quantize_rht col activation 8192x4096")
    xb = synth.make("activation")["x"]
    A = nv.rht_amax(dev_bf16(xb), axis="col", sign_seed=5)
    ra = np.float32(O.rht_amax(xb, axis=O.AXIS_COL, sign_seed=5))
    _same(A.cpu().numpy().view(np.uint32), np.array([ra]).view(np.uint32), "amax")
    q = nv.quantize_rht(dev_bf16(xb), A, axis="col", sign_seed=5)
    torch.cuda.synchronize()
    rc, rs, _ = O.quantize_rht(xb, ra, axis=O.AXIS_COL, sign_seed=5)
    _same(q.scales.cpu().numpy(), rs, "scales")
    _same(q.codes.cpu().numpy(), rc, "codes")


def test_full_gradient_col_rht_sr():
    """The other weight-gradient operand: the 16384x8192 gradient, column
    blocks after the transform, UE5M3 scales, stochastic rounding."""
    log("quantize_rht col SR gradient 16384x8192")
    xb = synth.make("gradient")["x"]
    A = nv.rht_amax(dev_bf16(xb), axis="col", sign_seed=9)
    ra = np.float32(O.rht_amax(xb, axis=O.AXIS_COL, sign_seed=9))
    _same(A.cpu().numpy().view(np.uint32), np.array([ra]).view(np.uint32), "amax")
    q = nv.quantize_rht(dev_bf16(xb), A, axis="col", sign_seed=9, fmt="ue5m3", select="6",
                        rounding="sr", seed=1234)
    torch.cuda.synchronize()
    rc, rs, _ = O.quantize_rht(xb, ra, axis=O.AXIS_COL, sign_seed=9, fmt=O.FMT_UE5M3,
                               select=O.SELECT_6, rounding=O.ROUND_SR, seed=1234)
    _same(q.scales.cpu().numpy(), rs, "scales")
    _same(q.codes.cpu().numpy(), rc, "codes")
