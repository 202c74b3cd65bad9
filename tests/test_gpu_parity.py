"""GPU-vs-oracle parity of every hot-path step through the C ABI: tensor amax,
row-wise / column-wise / fused quantization (E4M3 and UE5M3 scales, max->6,
Four-Over-Six, stochastic rounding), dequantization with the error report,
and fake-quant forward/backward (tied and dual scales).

Bar: packed codes, scale bytes, 4/6 counts and SR outputs bit-exact; binary32
outputs within relative 1e-5 (they are computed in the same order on both
sides, so they are expected to be identical and the exact-match count is
reported)."""
import numpy as np
import pytest

import oracle as O
from helpers import assert_close_rel, dev_bf16, dev_f32, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
nv = pytest.importorskip("nvfp4_block_scaled_02_amd")
from nvfp4_block_scaled_02_amd import synth  # noqa: E402

FMTS = {"e4m3": O.FMT_E4M3, "ue5m3": O.FMT_UE5M3}
SELS = {"6": O.SELECT_6, "4over6": O.SELECT_4OVER6}
RNDS = {"rne": O.ROUND_RNE, "sr": O.ROUND_SR}
# The error report: both sides take each residual x - x_hat in binary64 the
# same way and sum n non-negative terms in binary64, the oracle in index order
# and the device in its fixed blocked order.  Any order of summing n
# non-negative terms is within (n - 1) u of the exact sum (u = 2^-53), and the
# oracle rounds each square once more than the device's fma: the two reports
# differ by at most 3 n u relative.


def sse_rel(n):
    return 3.0 * n * 2.0 ** -53


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _amax_t(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def run_quantize(xb, amax, fmt="e4m3", select="4over6", rounding="rne", axes="row", seed=0,
                 global_max=0.0, count4=True):
    """The device quantizer through the C ABI.  count4=False takes the
    launches that do not count (their own launch shapes); the returned count
    is then None and assert_same_quant skips it."""
    x = dev_bf16(xb)
    q = nv.quantize(x, _amax_t(amax), fmt=fmt, select=select, rounding=rounding, axes=axes,
                    seed=seed, global_max=global_max, count4=count4)
    torch.cuda.synchronize()
    out = {k: getattr(q, k).cpu().numpy() for k in ("codes", "scales", "codes_t", "scales_t")
           if getattr(q, k) is not None}
    out["count4"] = int(q.count4.item()) if count4 else None
    return out


def oracle_quantize(xb, amax, fmt="e4m3", select="4over6", rounding="rne", axes="row", seed=0,
                    global_max=0.0):
    kw = dict(fmt=FMTS[fmt], select=SELS[select], rounding=RNDS[rounding], seed=seed,
              global_max=global_max or None)
    out = {"count4": 0}
    if axes in ("row", "both"):
        c, s, n = O.quantize(xb, amax, **kw)
        out.update(codes=c, scales=s)
        out["count4"] += n
    if axes in ("col", "both"):
        c, s, n = O.quantize_cols(xb, amax, **kw)
        out.update(codes_t=c, scales_t=s)
        out["count4"] += n
    return out


def assert_same_quant(got, ref, what):
    for k in ("codes", "scales", "codes_t", "scales_t"):
        if k in ref:
            g, r = got[k], ref[k]
            assert g.shape == r.shape, (what, k, g.shape, r.shape)
            bad = np.argwhere(g != r)
            assert bad.size == 0, f"{what}: {k} differ at {len(bad)} positions, first {bad[:4].tolist()}"
    if got["count4"] is not None:
        assert got["count4"] == ref["count4"], (what, got["count4"], ref["count4"])


# ---------------------------------------------------------------- amax
@pytest.mark.parametrize("name", ["weight-1k", "weight", "activation"])
def test_tensor_amax_configs(name):
    xb = synth.make(name)["x"]
    log(f"amax {name} {xb.shape}")
    a = nv.tensor_amax(dev_bf16(xb))
    assert a.item() == O.tensor_amax(xb)


@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 1000, 4097, 1000003])
def test_tensor_amax_ragged(n):
    xb = synth.random_bf16(1, max(n, 1), seed=n)[0, :n].copy()
    if n > 3:
        xb[n - 1] = synth.to_bf16_bits(np.array([-77.5]))[0]  # the max sits in the tail
    x = dev_bf16(xb) if n else torch.empty(0, dtype=torch.bfloat16, device="cuda")
    a = nv.tensor_amax(x)
    assert a.item() == (O.tensor_amax(xb) if n else 0.0)


def test_tensor_amax_nan_inf():
    xb = synth.random_bf16(64, 64, seed=3)
    xi = xb.copy()
    xi[5, 7] = 0xFF80  # -inf
    assert np.isinf(nv.tensor_amax(dev_bf16(xi)).item())
    xn = xi.copy()
    xn[60, 1] = 0x7FC1  # NaN
    assert np.isnan(nv.tensor_amax(dev_bf16(xn)).item())


# ---------------------------------------------------------------- quantize: page workloads
def test_config1_weight_1k_both_selections_and_dequantize():
    """256x1024 N(0,1) with 0.1% x20, alpha = amax/(6*448) for both runs, RNE."""
    xb = synth.make("weight-1k")["x"]
    A = float(O.tensor_amax(xb))
    for sel in ("6", "4over6"):
        got = run_quantize(xb, A, select=sel, global_max=448.0)
        ref = oracle_quantize(xb, A, select=sel, global_max=448.0)
        assert_same_quant(got, ref, f"weight-1k {sel}")
        xh, xb16, bs = O.dequantize(ref["codes"], ref["scales"], A, global_max=448.0,
                                    want_bf16=True, want_block_scale=True)
        gx, gbs, gsse = nv.dequantize(torch.from_numpy(got["codes"]).cuda(),
                                      torch.from_numpy(got["scales"]).cuda(), _amax_t(A),
                                      global_max=448.0, want_block_scale=True,
                                      x_ref=dev_bf16(xb))
        gb16 = nv.dequantize(torch.from_numpy(got["codes"]).cuda(),
                             torch.from_numpy(got["scales"]).cuda(), _amax_t(A), global_max=448.0,
                             out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert np.array_equal(gx.cpu().numpy(), xh)
        assert np.array_equal(gb16.view(torch.int16).cpu().numpy().view(np.uint16), xb16)
        assert np.array_equal(gbs.cpu().numpy(), bs)
        sse = O.sse(xb, xh)
        assert abs(gsse.item() - sse) <= sse_rel(xb.size) * sse
        log(f"weight-1k select={sel}: count4={got['count4']} MSE={sse / xb.size:.6g}")


def test_config2_weight_4096():
    xb = synth.make("weight")["x"]
    A = float(O.tensor_amax(xb))
    got = run_quantize(xb, A, select="4over6")
    ref = oracle_quantize(xb, A, select="4over6")
    assert_same_quant(got, ref, "weight 4096x4096 4/6")
    log(f"weight 4096^2: 4/6 chose max->4 in {got['count4']} of {got['scales'].size} blocks")


@pytest.mark.parametrize("name", ["weight", "activation"])
def test_full_size_4over6_without_count(name):
    """The non-counting launches at full size: 8192x4096 takes the two
    1024-lane workgroups per CU of the headline kernel, 4096x4096 too."""
    xb = synth.make(name)["x"]
    A = float(O.tensor_amax(xb))
    got = run_quantize(xb, A, select="4over6", count4=False)
    ref = oracle_quantize(xb, A, select="4over6")
    assert_same_quant(got, ref, f"{name} {xb.shape} 4/6 without count")


@pytest.mark.parametrize("rows,cols", [(17, 48), (3, 1040), (64, 16)])
def test_small_ragged_4over6_without_count(rows, cols):
    """Tensors whose block count leaves a partial group of 64 blocks, through
    the 256-lane launch that small tensors take."""
    rng = np.random.default_rng(rows * 1000 + cols)
    xb = synth.to_bf16_bits((rng.standard_normal((rows, cols)) * 3).astype(np.float32))
    A = float(O.tensor_amax(xb))
    assert_same_quant(run_quantize(xb, A, select="4over6", count4=False),
                      oracle_quantize(xb, A, select="4over6"), f"{rows}x{cols} 4/6 without count")


@pytest.mark.parametrize("select,rounding,fmt,count4", [("4over6", "rne", "e4m3", False),
                                                      ("4over6", "rne", "e4m3", True),
                                                      ("6", "sr", "ue5m3", False)])
def test_task_counter_with_partial_group(select, rounding, fmt, count4):
    """6151x4112: 24,700 whole groups of 64 blocks and a partial group of 7.
    On a 256-CU GPU this takes the 1024-lane launch with the workgroups'
    task counters (three or more groups per wavefront), so the partial group
    goes to whichever wavefront draws task nwhole."""
    rows, cols = 6151, 4112
    rng = np.random.default_rng(6151)
    xb = synth.to_bf16_bits((rng.standard_t(3, size=(rows, cols)) * 0.5).astype(np.float32))
    A = float(O.tensor_amax(xb))
    log(f"task counter {rows}x{cols} {select} {rounding} {fmt} count4={count4}")
    got = run_quantize(xb, A, fmt=fmt, select=select, rounding=rounding, seed=77, count4=count4)
    ref = oracle_quantize(xb, A, fmt=fmt, select=select, rounding=rounding, seed=77)
    assert_same_quant(got, ref, f"{rows}x{cols} {select} {rounding} {fmt}")


def test_config3_activation_8192x4096_with_mse():
    xb = synth.make("activation")["x"]
    x = dev_bf16(xb)
    amax = nv.tensor_amax(x)
    q = nv.quantize(x, amax, select="4over6", count4=True)
    xh, sse = nv.dequantize(q.codes, q.scales, amax, global_max=q.global_max, x_ref=x)
    torch.cuda.synchronize()
    A = float(O.tensor_amax(xb))
    assert amax.item() == A
    ref = oracle_quantize(xb, A, select="4over6")
    got = {"codes": q.codes.cpu().numpy(), "scales": q.scales.cpu().numpy(),
           "count4": int(q.count4.item())}
    assert_same_quant(got, ref, "activation 8192x4096 4/6")
    rx = O.dequantize(ref["codes"], ref["scales"], A)
    assert np.array_equal(xh.cpu().numpy(), rx)
    r_sse = O.sse(xb, rx)
    assert abs(sse.item() - r_sse) <= sse_rel(xb.size) * r_sse
    log(f"activation: MSE {r_sse / xb.size:.6g}, count4 {got['count4']}")


def test_config5_gradient_stale_amax_ue5m3_sr_both_axes():
    """16384x8192 gradients, stale amax 0.8 A (clipping), UE5M3, SR seed 1234,
    row-wise and column-wise in one fused pass; every output compared."""
    xb = synth.make("gradient")["x"]
    A = float(O.tensor_amax(xb))
    As = float(np.float32(0.8) * np.float32(A))
    log("gradient: generated, running GPU")
    got = run_quantize(xb, As, fmt="ue5m3", select="6", rounding="sr", axes="both", seed=1234)
    log("gradient: running oracle")
    ref = oracle_quantize(xb, As, fmt="ue5m3", select="6", rounding="sr", axes="both", seed=1234)
    assert_same_quant(got, ref, "gradient both axes")
    clipped = int((np.abs(O.as_f32(xb)) > As).sum())
    log(f"gradient: {clipped} elements above the stale amax")
    assert clipped > 0


# ---------------------------------------------------------------- quantize: option grid
SHAPES = [(16, 16), (32, 48), (80, 144), (208, 1040), (64, 2064), (1040, 64)]


@pytest.mark.parametrize("fmt", ["e4m3", "ue5m3"])
@pytest.mark.parametrize("select,rounding", [("6", "rne"), ("4over6", "rne"), ("6", "sr")])
@pytest.mark.parametrize("axes", ["row", "col", "both"])
def test_quantize_option_grid(fmt, select, rounding, axes):
    for i, (r, c) in enumerate(SHAPES):
        xb = synth.random_bf16(r, c, seed=100 + i, outlier_frac=0.01, outlier_mult=30)
        A = float(O.tensor_amax(xb))
        kw = dict(fmt=fmt, select=select, rounding=rounding, axes=axes, seed=(5 << 32) | 77)
        assert_same_quant(run_quantize(xb, A, **kw), oracle_quantize(xb, A, **kw),
                          f"{r}x{c} {kw}")


def test_ragged_tail_of_row_stream():
    # chunk counts that are not multiples of the 1024-chunk workgroup tile
    for rows, cols in [(1, 16), (3, 16), (129, 48), (1023, 16), (4099, 32)]:
        xb = synth.random_bf16(rows, cols, seed=rows)
        A = float(O.tensor_amax(xb))
        assert_same_quant(run_quantize(xb, A), oracle_quantize(xb, A), f"{rows}x{cols}")


def test_custom_global_max_and_seed_high_bits():
    xb = synth.random_bf16(64, 256, seed=8)
    A = float(O.tensor_amax(xb))
    for gm in (100.0, 448.0, 3000.0):
        for sel in ("6", "4over6"):
            assert_same_quant(run_quantize(xb, A, select=sel, global_max=gm),
                              oracle_quantize(xb, A, select=sel, global_max=gm), f"S_g {gm}")
    for seed in (0, 1234, (1 << 63) | 5):
        kw = dict(fmt="e4m3", select="6", rounding="sr", axes="both", seed=seed)
        assert_same_quant(run_quantize(xb, A, **kw), oracle_quantize(xb, A, **kw), f"seed {seed}")


# ---------------------------------------------------------------- edge cases
def test_zero_tensor_and_signed_zeros():
    xb = np.zeros((32, 64), np.uint16)
    xb[3, :] = 0x8000  # -0
    got = run_quantize(xb, 0.0, axes="both")
    ref = oracle_quantize(xb, 0.0, axes="both")
    assert_same_quant(got, ref, "zeros")
    assert np.all(got["scales"] == 0)


def _bf16_bits(v):
    return np.array([v], np.float32).view(np.uint32)[0] >> 16


@pytest.mark.parametrize("rows,cols,axes", [(48, 144, "both"), (48, 136, "col"), (80, 272, "both")])
@pytest.mark.parametrize("select,rounding,fmt", [("4over6", "rne", "e4m3"), ("6", "sr", "ue5m3")])
def test_partial_tiles_with_non_finite_edges(rows, cols, axes, select, rounding, fmt):
    """The strip walker loads a partial tile with addresses clamped to the
    tensor's last row and last 8-column chunk, so the chunks of the tile that
    lie outside the tensor repeat those edge values.  With NaN, infinity and
    the largest bf16 on the last row and in the last columns, the stored
    outputs and the 4/6 count must still be the oracle's: no block of the
    tensor mixes with the repeated copies."""
    rng = np.random.default_rng(rows * 1000 + cols)
    xb = synth.to_bf16_bits(rng.standard_normal((rows, cols)).astype(np.float32))
    xb[rows - 1, 5] = _bf16_bits(np.inf)
    xb[rows - 1, cols - 3] = _bf16_bits(np.nan)
    xb[rows - 3, cols - 1] = 0x7F7F  # largest finite bf16
    xb[rows - 1, cols - 20] = 0xFF80  # -inf
    A = 3.0  # a stale, finite outer amax: the edge values clip or give NaN blocks
    log(f"partial tiles {rows}x{cols} {axes} {select} {rounding} {fmt}")
    got = run_quantize(xb, A, fmt=fmt, select=select, rounding=rounding, axes=axes, seed=9,
                       count4=select == "4over6")
    ref = oracle_quantize(xb, A, fmt=fmt, select=select, rounding=rounding, axes=axes, seed=9)
    assert_same_quant(got, ref, f"partial tiles {rows}x{cols} {axes}")


def test_partial_2d_tiles_with_non_finite_edges():
    """The same for 16x16 tile scales: a NaN and an infinity on the last row
    of a ragged tensor reach only their own tiles."""
    rows, cols = 48, 144
    rng = np.random.default_rng(3)
    xb = synth.to_bf16_bits(rng.standard_normal((rows, cols)).astype(np.float32))
    xb[rows - 1, 3] = _bf16_bits(np.inf)
    xb[rows - 1, cols - 2] = _bf16_bits(np.nan)
    a = 4.0
    q = nv.quantize_2d(dev_bf16(xb), _amax_t(a))
    torch.cuda.synchronize()
    got = [q.codes.cpu().numpy(), q.scales.cpu().numpy(), q.codes_t.cpu().numpy(),
           q.scales_t.cpu().numpy()]
    ref = O.quantize_2d(xb, a)
    for g, r, k in zip(got, ref, ("codes", "scales", "codes_t", "scales_t")):
        assert np.array_equal(g, r), k


@pytest.mark.parametrize("bad", [float("nan"), float("inf"), -1.0])
def test_unusable_amax_gives_nan_scales(bad):
    xb = synth.random_bf16(32, 64, seed=2)
    for fmt in ("e4m3", "ue5m3"):
        got = run_quantize(xb, bad, fmt=fmt, axes="both")
        assert_same_quant(got, oracle_quantize(xb, bad, fmt=fmt, axes="both"), f"amax {bad}")
        assert np.all(got["codes"] == 0)


def test_nan_and_inf_elements():
    xb = synth.random_bf16(32, 64, seed=4)
    xb[1, 3] = 0x7FC0  # NaN
    xb[2, 20] = 0x7F80  # +inf
    xb[17, 40] = 0xFF80  # -inf
    A = 50.0
    for sel in ("6", "4over6"):
        for fmt in ("e4m3", "ue5m3"):
            kw = dict(fmt=fmt, select=sel, axes="both")
            assert_same_quant(run_quantize(xb, A, **kw), oracle_quantize(xb, A, **kw),
                              f"nan/inf {kw}")


def test_denormal_and_extreme_magnitudes():
    rng = np.random.default_rng(6)
    tiny = synth.to_bf16_bits(rng.standard_normal((32, 64)) * 1e-39)  # bf16 subnormals
    huge = synth.to_bf16_bits(rng.standard_normal((32, 64)) * 1e38)
    mixed = synth.to_bf16_bits(rng.standard_normal((32, 64)) * np.exp(rng.uniform(-80, 80, (32, 64))))
    for name, xb in [("tiny", tiny), ("huge", huge), ("mixed", mixed)]:
        A = float(O.tensor_amax(xb))
        for kw in [dict(select="6"), dict(select="4over6"), dict(fmt="ue5m3", select="6"),
                   dict(select="6", rounding="sr", axes="both", seed=9)]:
            assert_same_quant(run_quantize(xb, A, **kw), oracle_quantize(xb, A, **kw),
                              f"{name} {kw}")


def test_determinism():
    """Three runs of each output are bitwise identical: the quantizers (both
    layouts, the 4/6 count), the dequantized values and the squared-error
    report (a fixed-order grid sum), and the fake-quant forward and backward
    (tied and dual)."""
    xb = synth.make("weight-1k")["x"]
    A = float(O.tensor_amax(xb))
    runs = [run_quantize(xb, A, axes="both") for _ in range(3)]
    for r in runs[1:]:
        for k in ("codes", "scales", "codes_t", "scales_t"):
            assert np.array_equal(r[k], runs[0][k])
        assert r["count4"] == runs[0]["count4"]
    xa = synth.make("activation")["x"]
    x = dev_bf16(xa)
    amax = nv.tensor_amax(x)
    q = nv.quantize(x, amax, select="4over6")
    reps = []
    for _ in range(3):
        xh, sse = nv.dequantize(q.codes, q.scales, amax, global_max=q.global_max, x_ref=x)
        torch.cuda.synchronize()
        reps.append((xh.cpu().numpy(), sse.cpu().numpy().view(np.uint64)[0]))
    for xh, bits in reps[1:]:
        assert np.array_equal(xh, reps[0][0])
        assert bits == reps[0][1], "the squared-error report changed between runs"
    xw = dev_bf16(xb)
    s = torch.from_numpy(O.dequantize(runs[0]["codes"], runs[0]["scales"], A,
                                      want_block_scale=True)[1]).cuda()
    s2 = s * 1.125
    g = torch.from_numpy(np.random.default_rng(5).standard_normal(xb.shape).astype(np.float32)).cuda()
    outs = []
    for _ in range(3):
        o = [nv.fakequant_fwd(xw, s), nv.fakequant_fwd(xw, s, s2), *nv.fakequant_bwd(xw, g, s),
             *nv.fakequant_bwd(xw, g, s, s2)]
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in o])
    for o in outs[1:]:
        for a, b in zip(o, outs[0]):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ---------------------------------------------------------------- dequantize
@pytest.mark.parametrize("fmt", ["e4m3", "ue5m3"])
def test_dequantize_every_code(fmt):
    """Every nibble under every scale byte (NaN codes included)."""
    nsc = 256
    codes = np.tile(np.arange(256, dtype=np.uint8), (nsc, 1))  # [256, 256] -> 512 cols
    scales = np.repeat(np.arange(nsc, dtype=np.uint8)[:, None], 32, axis=1)
    A, gm = 3.0, 448.0
    ref, ref16, refbs = O.dequantize(codes, scales, A, fmt=FMTS[fmt], global_max=gm,
                                     want_bf16=True, want_block_scale=True)
    cd, sd = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    got, gbs = nv.dequantize(cd, sd, _amax_t(A), global_max=gm, fmt=fmt, want_block_scale=True)
    g16 = nv.dequantize(cd, sd, _amax_t(A), global_max=gm, fmt=fmt, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    g = got.cpu().numpy()
    assert np.array_equal(np.isnan(g), np.isnan(ref))
    assert np.array_equal(g[~np.isnan(ref)], ref[~np.isnan(ref)])
    gb = g16.view(torch.int16).cpu().numpy().view(np.uint16)
    nan16 = (ref16 & 0x7FFF) > 0x7F80
    assert np.array_equal((gb & 0x7FFF) > 0x7F80, nan16)
    assert np.array_equal(gb[~nan16], ref16[~nan16])
    bs = gbs.cpu().numpy()
    assert np.array_equal(np.isnan(bs), np.isnan(refbs))
    assert np.array_equal(bs[~np.isnan(refbs)], refbs[~np.isnan(refbs)])


# ---------------------------------------------------------------- fake quantization
def _fq_case(xb, g, s_pre, s_post=None):
    x = dev_bf16(xb)
    gd = dev_f32(g)
    sp = dev_f32(s_pre)
    so = None if s_post is None else dev_f32(s_post)
    xq = nv.fakequant_fwd(x, sp, so)
    bw = nv.fakequant_bwd(x, gd, sp, so)
    torch.cuda.synchronize()
    rq = O.fakequant_fwd(xb, s_pre, s_post)
    rb = O.fakequant_bwd(xb, g, s_pre, s_post)
    assert np.array_equal(xq.cpu().numpy(), rq), "x~ differs"
    assert np.array_equal(bw[0].cpu().numpy(), rb[0]), "dL/dx differs"
    exact = 0
    for got, ref, nm in zip(bw[1:], rb[1:], ("ds_pre", "ds_post")):
        gn = got.cpu().numpy()
        assert_close_rel(gn, ref, 1e-5, nm)
        exact += int(np.count_nonzero(gn == ref))
    return exact, sum(r.size for r in rb[1:])


def test_config4_scale_learning_step():
    """14336x4096 weight, scales initialised as amax/6 in E4M3 (two-level, S_g
    448), tied and dual scales, dual with s_post perturbed by 1.125."""
    d = synth.make("qat")
    xb, g = d["x"], d["g"]
    A = float(O.tensor_amax(xb))
    codes, scales, _ = O.quantize(xb, A, select=O.SELECT_6, global_max=448.0)
    s = O.dequantize(codes, scales, A, global_max=448.0, want_block_scale=True)[1]
    # the GPU path reaches the same initial scales
    x = dev_bf16(xb)
    q = nv.quantize(x, _amax_t(A), select="6", global_max=448.0)
    _, gs = nv.dequantize(q.codes, q.scales, _amax_t(A), global_max=448.0, want_block_scale=True)
    assert np.array_equal(gs.cpu().numpy(), s)
    del x, q, gs
    for s_post in (None, s, (s * np.float32(1.125)).astype(np.float32)):
        exact, tot = _fq_case(xb, g, s, s_post)
        log(f"qat s_post={'tied' if s_post is None else 'dual'}: {exact}/{tot} scale gradients bit-identical")


def test_fakequant_edges():
    rng = np.random.default_rng(11)
    xb = synth.random_bf16(48, 64, seed=12)
    x = O.as_f32(xb)
    g = rng.standard_normal((48, 64)).astype(np.float32)
    s = (np.abs(x).reshape(48, 4, 16).max(2) / 6).astype(np.float32)
    s[0, 0] = 0.0  # zero scale
    s[1, 1] *= 0.1  # clamp active
    s[2, 2] = 1e-38  # reciprocal near overflow
    s[3, 3] = 1e-45  # reciprocal overflows
    _fq_case(xb, g, s)
    _fq_case(xb, g, s, (s * 1.5).astype(np.float32))
    # ragged: a single block row and a tail of quads
    xb1 = synth.random_bf16(1, 16, seed=13)
    g1 = rng.standard_normal((1, 16)).astype(np.float32)
    s1 = np.array([[0.1]], np.float32)
    _fq_case(xb1, g1, s1)
    _fq_case(xb1, g1, s1, s1 * 2)
