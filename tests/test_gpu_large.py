"""GPU-vs-oracle parity at the largest sizes: a 65536 x 65552 bf16 tensor
(4,296,015,872 elements, past 2^32), where element indices, the counter
hash's high word and every 64-bit address computation are exercised.

The tensor is generated on the GPU from a seeded generator in row chunks
(8.6 GB).  The oracle recomputes sampled rows and sampled column strips
(blocks are independent given the outer scale, and SR variates depend
only on the element's index), with the rows' and columns' positions in the
whole tensor: row 65520 holds element index 2^32 at column 256 (the hash
key changes inside the row), columns 65536.. hold the column-wise indices
past 2^32, and the last 128-column strip holds only 16 columns.

The tensor amax is pinned by a planted maximum and a planted NaN past index
2^32 (the property that holds at any size); the quantizers take a given
(stale) outer amax, so no oracle input comes from the GPU.  The
re-quantization takes a seeded random NVFP4 source of the same shape.

Bar: codes and scale bytes bit-exact; dequantized values bit-exact."""
import numpy as np
import pytest

import oracle as O
from helpers import log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
nv = pytest.importorskip("nvfp4_block_scaled_02_amd")

ROWS, COLS = 65536, 65552
BOUNDARY_ROW = (1 << 32) // COLS  # 65520: element 2^32 lies in this row
SAMPLE_ROWS = [0, 1, 40000, BOUNDARY_ROW - 1, BOUNDARY_ROW, BOUNDARY_ROW + 1, ROWS - 1]
SAMPLE_COL0 = [0, 32768, 65536]  # 16-column strips; the last is past index 2^32
A_STALE = np.float32(4.0)        # |x| > 4 saturates (stale outer amax)


@pytest.fixture(scope="module")
def big():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    free, _ = torch.cuda.mem_get_info()
    if free < 40 * 2 ** 30:
        pytest.skip("needs 40 GiB of free device memory")
    assert BOUNDARY_ROW * COLS < (1 << 32) < (BOUNDARY_ROW + 1) * COLS
    log(f"generating {ROWS}x{COLS} bf16 on the device")
    g = torch.Generator(device="cuda")
    g.manual_seed(20260101)
    x = torch.empty((ROWS, COLS), dtype=torch.bfloat16, device="cuda")
    step = 2048
    for r in range(0, ROWS, step):
        x[r:r + step] = torch.randn((step, COLS), generator=g, device="cuda", dtype=torch.float32)
    torch.cuda.synchronize()
    yield x
    del x
    torch.cuda.empty_cache()


def _rows_host(x, rows):
    return np.stack([x[r].view(torch.int16).cpu().numpy().view(np.uint16) for r in rows])


def _strip_host(x, c0):
    return np.ascontiguousarray(x[:, c0:c0 + 16].view(torch.int16).cpu().numpy().view(np.uint16))


def _same(got, ref, what):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{what}: differ at {len(bad)} positions, first {bad[:4].tolist()}"


def test_amax_planted_past_2_32(big):
    """The grid-stride amax over 4.3e9 elements finds a maximum planted at
    an index past 2^32 (all other values are N(0,1) draws, far below it),
    and a NaN planted there makes the result NaN."""
    x = big
    r, c = ROWS - 3, COLS - 5
    saved = x[r, c].clone()
    try:
        x[r, c] = 1000.0
        a = nv.tensor_amax(x)
        torch.cuda.synchronize()
        assert float(a.item()) == 1000.0
        x[r, c] = float("nan")
        a = nv.tensor_amax(x)
        torch.cuda.synchronize()
        assert np.isnan(float(a.item()))
    finally:
        x[r, c] = saved
    log("amax planted max / NaN past 2^32: ok")


def test_sr_fused_rows_and_cols_past_2_32(big):
    """Gradient-style quantization: UE5M3, max->6, stochastic rounding,
    row-wise and column-wise in one fused pass, stale outer amax."""
    x = big
    amax = torch.tensor([A_STALE], dtype=torch.float32, device="cuda")
    log("fused SR quantize 65536x65552")
    q = nv.quantize(x, amax, fmt="ue5m3", select="6", rounding="sr", axes="both", seed=1234)
    torch.cuda.synchronize()
    xr = _rows_host(x, SAMPLE_ROWS)
    for i, r in enumerate(SAMPLE_ROWS):
        rc, rs, _ = O.quantize(xr[i:i + 1], A_STALE, fmt=O.FMT_UE5M3, select=O.SELECT_6,
                               rounding=O.ROUND_SR, seed=1234, row0=r)
        _same(q.scales[r:r + 1].cpu().numpy(), rs, f"row scales, row {r}")
        _same(q.codes[r:r + 1].cpu().numpy(), rc, f"row codes, row {r}")
    for c0 in SAMPLE_COL0:
        xs = _strip_host(x, c0)
        rct, rst, _ = O.quantize_cols(xs, A_STALE, col0=c0, fmt=O.FMT_UE5M3, select=O.SELECT_6,
                                      rounding=O.ROUND_SR, seed=1234)
        _same(q.scales_t[c0:c0 + 16].cpu().numpy(), rst, f"column scales, strip {c0}")
        _same(q.codes_t[c0:c0 + 16].cpu().numpy(), rct, f"column codes, strip {c0}")
    del q
    log("fused SR past 2^32: ok")


def test_4over6_rows_and_dequantize_past_2_32(big):
    """Activation-style quantization (E4M3, Four-Over-Six, RNE) and its
    dequantization to bf16 at the same size."""
    x = big
    amax = torch.tensor([A_STALE], dtype=torch.float32, device="cuda")
    log("4/6 quantize 65536x65552")
    q = nv.quantize(x, amax, select="4over6")
    gm = O.default_global_max(O.FMT_E4M3, O.SELECT_4OVER6)
    xh = nv.dequantize(q.codes, q.scales, amax, global_max=gm, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    xr = _rows_host(x, SAMPLE_ROWS)
    for i, r in enumerate(SAMPLE_ROWS):
        rc, rs, _ = O.quantize(xr[i:i + 1], A_STALE, select=O.SELECT_4OVER6, row0=r)
        _same(q.scales[r:r + 1].cpu().numpy(), rs, f"scales, row {r}")
        _same(q.codes[r:r + 1].cpu().numpy(), rc, f"codes, row {r}")
        _, ref_bf16 = O.dequantize(rc, rs, A_STALE, select=O.SELECT_4OVER6, want_bf16=True)
        got = xh[r:r + 1].view(torch.int16).cpu().numpy().view(np.uint16)
        _same(got, ref_bf16, f"x_hat bf16, row {r}")
    del q, xh
    log("4/6 + dequantize past 2^32: ok")


def test_rowscaled_sr_past_2_32(big):
    """Per-row outer scales with stochastic rounding (WIDE hash path of the
    row-scaled quantizer); the row amaxes are a seeded input, stale for
    some rows."""
    x = big
    ra = np.random.default_rng(7).uniform(1.0, 6.0, ROWS).astype(np.float32)
    log("row-scaled SR quantize 65536x65552")
    q = nv.quantize_rowscaled(x, torch.from_numpy(ra).cuda(), fmt="ue5m3", select="6",
                              rounding="sr", seed=99)
    torch.cuda.synchronize()
    xr = _rows_host(x, SAMPLE_ROWS)
    for i, r in enumerate(SAMPLE_ROWS):
        rc, rs, _ = O.quantize_rowscaled(xr[i:i + 1], ra[r:r + 1], fmt=O.FMT_UE5M3,
                                         select=O.SELECT_6, rounding=O.ROUND_SR, seed=99, row0=r)
        _same(q.scales[r:r + 1].cpu().numpy(), rs, f"scales, row {r}")
        _same(q.codes[r:r + 1].cpu().numpy(), rc, f"codes, row {r}")
    del q
    log("row-scaled SR past 2^32: ok")


def test_pertoken_sr_past_2_32(big):
    """The one-launch per-token quantizer past element 2^32 (its WIDE hash
    path): the same memory viewed as rows of 4096 columns, the longest rows
    it takes in one launch."""
    x = big.view(-1, 4096)
    rows = x.shape[0]
    first_wide = (1 << 32) // 4096  # the first row whose indices pass 2^32
    sample = [0, 1, first_wide - 1, first_wide, first_wide + 1, rows - 1]
    log(f"per-token SR quantize {rows}x4096")
    q = nv.quantize_pertoken(x, fmt="ue5m3", select="6", rounding="sr", seed=77)
    torch.cuda.synchronize()
    xr = _rows_host(x, sample)
    for i, r in enumerate(sample):
        ra = O.row_amax(xr[i:i + 1])
        _same(q.amax[r:r + 1].cpu().numpy().view(np.uint32), ra.view(np.uint32),
              f"row amax, row {r}")
        rc, rs, _ = O.quantize_rowscaled(xr[i:i + 1], ra, fmt=O.FMT_UE5M3, select=O.SELECT_6,
                                         rounding=O.ROUND_SR, seed=77, row0=r)
        _same(q.scales[r:r + 1].cpu().numpy(), rs, f"scales, row {r}")
        _same(q.codes[r:r + 1].cpu().numpy(), rc, f"codes, row {r}")
    del q
    log("per-token SR past 2^32: ok")


def _rand_u8(shape, lo, hi, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randint(lo, hi, shape, generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)


@pytest.mark.parametrize("target", ["mxfp8", "nvfp4"])
def test_requant_past_2_32(target):
    """Dequantize -> transpose -> SR re-quantize of a 65536x65552 NVFP4
    tensor (seeded random codes and finite E4M3 scale bytes, given outer
    amaxes): the oracle recomputes 16-column source strips, including the
    last (output rows whose indices pass 2^32), with their output offset."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if torch.cuda.mem_get_info()[0] < 24 * 2 ** 30:
        pytest.skip("needs 24 GiB of free device memory")
    log(f"requant {target} 65536x65552")
    codes = _rand_u8((ROWS, COLS // 2), 0, 256, 31)
    scales = _rand_u8((ROWS, COLS // 16), 0x20, 0x60, 32)
    amax = torch.tensor([100.0], dtype=torch.float32, device="cuda")
    gm = O.default_global_max(O.FMT_E4M3, O.SELECT_4OVER6)
    kw = {"dst_amax": torch.tensor([20.0], dtype=torch.float32, device="cuda")} if target == "nvfp4" else {}
    out, out_s = nv.requantize_t(codes, scales, amax=amax, global_max=gm, target=target, seed=4242, **kw)
    torch.cuda.synchronize()
    for c0 in SAMPLE_COL0:
        cs = np.ascontiguousarray(codes[:, c0 // 2:c0 // 2 + 8].cpu().numpy())
        ss = np.ascontiguousarray(scales[:, c0 // 16:c0 // 16 + 1].cpu().numpy())
        okw = {"dst_amax": 20.0} if target == "nvfp4" else {}
        ro, rs = O.requant_t(cs, ss, amax=100.0, global_max=gm, target=target, seed=4242, col0=c0,
                             **okw)
        _same(out_s[c0:c0 + 16].cpu().numpy(), rs, f"{target} scales_t, strip {c0}")
        _same(out[c0:c0 + 16].cpu().numpy(), ro, f"{target} out_t, strip {c0}")
    del out, out_s, codes, scales
    torch.cuda.empty_cache()
    log(f"requant {target} past 2^32: ok")


def test_rht_sr_past_2_32(big):
    """The random Hadamard transform before SR quantization (UE5M3, max->6),
    column blocks (the weight-gradient operand) and row blocks."""
    x = big
    amax = torch.tensor([A_STALE], dtype=torch.float32, device="cuda")
    kw = dict(sign_seed=17, fmt="ue5m3", select="6", rounding="sr", seed=777)
    okw = dict(sign_seed=17, fmt=O.FMT_UE5M3, select=O.SELECT_6, rounding=O.ROUND_SR, seed=777)
    log("RHT column SR 65536x65552")
    q = nv.quantize_rht(x, amax, axis="col", **kw)
    torch.cuda.synchronize()
    for c0 in SAMPLE_COL0:
        rc, rs, _ = O.quantize_rht(_strip_host(x, c0), A_STALE, axis=O.AXIS_COL, out_row0=c0, **okw)
        _same(q.scales[c0:c0 + 16].cpu().numpy(), rs, f"RHT column scales, strip {c0}")
        _same(q.codes[c0:c0 + 16].cpu().numpy(), rc, f"RHT column codes, strip {c0}")
    del q
    log("RHT row SR 65536x65552")
    q = nv.quantize_rht(x, amax, axis="row", **kw)
    torch.cuda.synchronize()
    xr = _rows_host(x, SAMPLE_ROWS)
    for i, r in enumerate(SAMPLE_ROWS):
        rc, rs, _ = O.quantize_rht(xr[i:i + 1], A_STALE, axis=O.AXIS_ROW, out_row0=r, **okw)
        _same(q.scales[r:r + 1].cpu().numpy(), rs, f"RHT row scales, row {r}")
        _same(q.codes[r:r + 1].cpu().numpy(), rc, f"RHT row codes, row {r}")
    del q
    log("RHT SR past 2^32: ok")
