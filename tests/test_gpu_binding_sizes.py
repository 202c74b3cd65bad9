"""The Python binding checks every buffer against the extent the kernels
index and raises before any launch (the C ABI sees only pointers).  Each
case passes one wrongly sized tensor; nothing reaches the GPU kernels."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
nv = pytest.importorskip("nvfp4_block_scaled_02_amd")


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8, device="cuda")


def _f32(*shape):
    return torch.zeros(shape, dtype=torch.float32, device="cuda")


def test_quantize_outputs():
    x = torch.zeros((32, 64), dtype=torch.bfloat16, device="cuda")
    a = _f32(1)
    bad = [dict(codes=_u8(32, 31)), dict(scales=_u8(32, 3)), dict(count4=torch.zeros(2, dtype=torch.int64, device="cuda"))]
    for out in bad:
        with pytest.raises(ValueError):
            nv.quantize(x, a, out=out)
    with pytest.raises(ValueError):
        nv.quantize(x, a, axes="col", out=dict(codes_t=_u8(64, 15)))
    with pytest.raises(ValueError):
        nv.quantize(x, a, axes="both", out=dict(scales_t=_u8(64, 3)))
    with pytest.raises(ValueError):
        nv.quantize(x, _f32(2))
    with pytest.raises(ValueError):
        nv.quantize(x, a, count4=True, workspace=_u8(100))


def test_dequantize_buffers():
    c, s, a = _u8(32, 32), _u8(32, 4), _f32(1)
    with pytest.raises(ValueError):
        nv.dequantize(c, _u8(32, 3), a, global_max=448.0)
    with pytest.raises(ValueError):
        nv.dequantize(c, s, a, global_max=448.0, out=_f32(32, 63))
    with pytest.raises(ValueError):
        nv.dequantize(c, s, a, global_max=448.0,
                      x_ref=torch.zeros((32, 60), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        nv.dequantize_rowscaled(c, s, _f32(31), global_max=448.0)


def test_fakequant_buffers():
    x = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    s = _f32(16, 4)
    with pytest.raises(ValueError):
        nv.fakequant_fwd(x, _f32(16, 3))
    with pytest.raises(ValueError):
        nv.fakequant_fwd(x, s, _f32(15, 4))
    with pytest.raises(ValueError):
        nv.fakequant_fwd(x, s, out=_f32(16, 63))
    with pytest.raises(ValueError):
        nv.fakequant_bwd(x, _f32(16, 60), s)
    with pytest.raises(ValueError):
        nv.fakequant_bwd(x, _f32(16, 64), s, out=dict(ds_pre=_f32(8)))
    with pytest.raises(ValueError):
        nv.fakequant_bwd(x, _f32(16, 64), s, s, out=dict(ds_post=_f32(3)))


def test_requantize_and_amax_buffers():
    c, s, a = _u8(64, 16), _u8(64, 2), _f32(1)
    with pytest.raises(ValueError):
        nv.requantize_t(c, s, amax=a, global_max=448.0, target="mxfp8", out=dict(out_t=_u8(32, 63)))
    with pytest.raises(ValueError):
        nv.requantize_t(c, s, amax=a, global_max=448.0, target="nvfp4", dst_amax=a,
                        out=dict(scales_t=_u8(32, 3)))
    with pytest.raises(ValueError):
        nv.dequantized_amax(c, s, row_amaxes=_f32(63), global_max=448.0)
    with pytest.raises(ValueError):
        nv.tensor_amax(torch.zeros(64, dtype=torch.bfloat16, device="cuda"), out=_f32(2))
    with pytest.raises(ValueError):
        nv.row_amax(torch.zeros((8, 32), dtype=torch.bfloat16, device="cuda"), out=_f32(7))
    x = torch.zeros((32, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        nv.quantize_rht(x, a, axis="col", out=dict(codes=_u8(32, 31)))
    with pytest.raises(ValueError):
        nv.quantize_2d(x, a, out=dict(codes_t=_u8(64, 15)))
