"""GPU-vs-oracle parity, through the C ABI, of the other block-scale
selection rules (Four-Over-Six by absolute error and by largest error; the
MSE scale sweep over every scale code) on every quantization path, and of
the amax-parameterized fake quantization.

Bar: codes, scale bytes and counts bit-exact; binary32 outputs bit-exact
(their tolerance, relative 1e-5, is not needed: the arithmetic is the same)."""
import numpy as np
import pytest

import oracle as O
from helpers import dev_bf16, dev_f32, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
nv = pytest.importorskip("nvfp4_block_scaled_02_amd")
from nvfp4_block_scaled_02_amd import synth  # noqa: E402

SELS = {"4over6-mae": O.SELECT_4OVER6_MAE, "4over6-maxerr": O.SELECT_4OVER6_MAXERR,
        "sweep": O.SELECT_SWEEP}
FMTS = {"e4m3": O.FMT_E4M3, "ue5m3": O.FMT_UE5M3}


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _same(got, ref, what):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{what}: differ at {len(bad)} positions, first {bad[:4].tolist()}"


def _tensor(rows, cols, seed, spread=1.5):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)) * np.exp(rng.normal(0, spread, (rows, 1)))
    x[rng.random((rows, cols)) < 0.01] *= 30
    return synth.to_bf16_bits(x.astype(np.float32))


def _gpu_q(xb, amax, select, fmt="e4m3", axes="row"):
    q = nv.quantize(dev_bf16(xb), dev_f32(np.array([amax], np.float32)), fmt=fmt, select=select,
                    axes=axes, count4=True)
    torch.cuda.synchronize()
    cpu = lambda t: None if t is None else t.cpu().numpy()
    return cpu(q.codes), cpu(q.scales), cpu(q.codes_t), cpu(q.scales_t), int(q.count4.item())


# ---------------------------------------------------------------- row-wise, per tensor
@pytest.mark.parametrize("select", ["4over6-mae", "4over6-maxerr"])
def test_rules_full_activation(select):
    log(f"rule {select} activation 8192x4096")
    xb = synth.make("activation")["x"]
    A = O.tensor_amax(xb)
    c, s, _, _, n = _gpu_q(xb, A, select)
    rc, rs, rn = O.quantize(xb, A, select=SELS[select])
    _same(s, rs, "scales")
    _same(c, rc, "codes")
    assert n == rn


@pytest.mark.parametrize("select", ["4over6-mae", "4over6-maxerr", "sweep"])
@pytest.mark.parametrize("rows,cols", [(1, 16), (7, 48), (33, 1040), (256, 1024), (5, 4112)])
def test_rules_row_shapes(select, rows, cols):
    log(f"rule {select} {rows}x{cols}")
    xb = _tensor(rows, cols, rows * 3 + cols)
    A = O.tensor_amax(xb)
    c, s, _, _, n = _gpu_q(xb, A, select)
    rc, rs, rn = O.quantize(xb, A, select=SELS[select])
    _same(s, rs, "scales")
    _same(c, rc, "codes")
    assert n == rn


def test_sweep_full_activation_sampled_rows():
    """The sweep at 8192x4096 on the GPU; the oracle recomputes 64 sampled
    rows (rows are independent given the tensor's outer scale)."""
    log("sweep activation 8192x4096 (sampled rows)")
    xb = synth.make("activation")["x"]
    A = O.tensor_amax(xb)
    c, s, _, _, _ = _gpu_q(xb, A, "sweep")
    rows = np.random.default_rng(5).choice(xb.shape[0], 64, replace=False)
    rc, rs, _ = O.quantize(np.ascontiguousarray(xb[rows]), A, select=O.SELECT_SWEEP)
    _same(s[rows], rs, "sweep scales (sampled rows)")
    _same(c[rows], rc, "sweep codes (sampled rows)")


def test_sweep_ue5m3_and_stale_amax():
    xb = _tensor(64, 512, 9)
    A = np.float32(O.tensor_amax(xb) * 0.5)  # stale: the largest blocks saturate
    for fmt in ("e4m3", "ue5m3"):
        c, s, _, _, _ = _gpu_q(xb, A, "sweep", fmt=fmt)
        rc, rs, _ = O.quantize(xb, A, fmt=FMTS[fmt], select=O.SELECT_SWEEP)
        _same(s, rs, f"sweep scales {fmt}")
        _same(c, rc, f"sweep codes {fmt}")


# ---------------------------------------------------------------- column-wise / fused
@pytest.mark.parametrize("select", ["4over6-mae", "4over6-maxerr", "sweep"])
@pytest.mark.parametrize("rows,cols", [(32, 128), (48, 208), (160, 272)])
def test_rules_fused_row_and_col(select, rows, cols):
    log(f"rule {select} fused {rows}x{cols}")
    xb = _tensor(rows, cols, rows + 7 * cols)
    A = O.tensor_amax(xb)
    c, s, ct, st, n = _gpu_q(xb, A, select, axes="both")
    rc, rs, rn = O.quantize(xb, A, select=SELS[select])
    rct, rst, rnt = O.quantize_cols(xb, A, select=SELS[select])
    _same(s, rs, "scales")
    _same(c, rc, "codes")
    _same(st, rst, "scales_t")
    _same(ct, rct, "codes_t")
    assert n == rn + rnt


# ---------------------------------------------------------------- per-row outer scales
@pytest.mark.parametrize("select", ["4over6-mae", "4over6-maxerr", "sweep"])
@pytest.mark.parametrize("rows,cols", [(5, 48), (19, 1040), (6, 4096)])
def test_rules_rowscaled(select, rows, cols):
    log(f"rule {select} rowscaled {rows}x{cols}")
    xb = _tensor(rows, cols, 2 * rows + cols)
    ra = O.row_amax(xb)
    q = nv.quantize_rowscaled(dev_bf16(xb), dev_f32(ra), select=select, count4=True)
    torch.cuda.synchronize()
    rc, rs, rn = O.quantize_rowscaled(xb, ra, select=SELS[select])
    _same(q.scales.cpu().numpy(), rs, "scales")
    _same(q.codes.cpu().numpy(), rc, "codes")
    assert int(q.count4.item()) == rn


# ---------------------------------------------------------------- amax-parameterized fake quant
def _amaxes(xb, seed):
    rng = np.random.default_rng(seed)
    a = np.abs(O.as_f32(xb)).reshape(-1, 16).max(axis=1) * rng.uniform(0.8, 1.2, xb.size // 16)
    a[::97] = 0.0  # zero amax: zero scale
    return a.astype(np.float32).reshape(xb.shape[0], xb.shape[1] // 16)


@pytest.mark.parametrize("rows,cols,dual", [(64, 256, False), (64, 256, True),
                                            (14336, 4096, False), (14336, 4096, True)])
def test_fakequant_amax(rows, cols, dual):
    log(f"fakequant amax {rows}x{cols} dual={dual}")
    if rows == 14336:
        d = synth.make("qat")
        xb, g = d["x"], d["g"]
    else:
        xb = _tensor(rows, cols, 3, spread=0.5)
        g = (np.random.default_rng(4).standard_normal((rows, cols)) * 1e-3).astype(np.float32)
    a = _amaxes(xb, 6)
    ap = (a * np.float32(1.125)).astype(np.float32) if dual else None
    x_d, g_d, a_d = dev_bf16(xb), dev_f32(g), dev_f32(a)
    ap_d = dev_f32(ap) if dual else None
    xq = nv.fakequant_fwd(x_d, a_d, ap_d, amax=True)
    res = nv.fakequant_bwd(x_d, g_d, a_d, ap_d, amax=True)
    torch.cuda.synchronize()
    rxq = O.fakequant_fwd(xb, a, ap, amax=True)
    rres = O.fakequant_bwd(xb, g, a, ap, amax=True)
    _same(xq.cpu().numpy().view(np.uint32), rxq.view(np.uint32), "x~")
    for got, ref, what in zip(res, rres, ("dx", "da_pre", "da_post")):
        _same(got.cpu().numpy().view(np.uint32), ref.view(np.uint32), what)
