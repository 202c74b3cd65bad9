"""nvfp4_tensor_amax_noalloc (the library's static scratch in place of a
workspace) against nvfp4_tensor_amax (a caller's workspace), through the C
ABI: two calls in a row, the second on a smaller input, each bit-exact
against the workspace entry point on the same input."""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
nv = pytest.importorskip("nvfp4_block_scaled_02_amd")
from nvfp4_block_scaled_02_amd import _native as N  # noqa: E402
from nvfp4_block_scaled_02_amd import synth  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _amax_both(x):
    lib = N.lib()
    s = torch.cuda.current_stream().cuda_stream
    ws = torch.zeros(N.WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    a_ws = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    a_na = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    assert lib.nvfp4_tensor_amax(x.data_ptr(), x.numel(), a_ws.data_ptr(), ws.data_ptr(), s) == N.OK
    assert lib.nvfp4_tensor_amax_noalloc(x.data_ptr(), x.numel(), a_na.data_ptr(), s) == N.OK
    torch.cuda.synchronize()
    return (a_ws.cpu().numpy().view(np.uint32)[0], a_na.cpu().numpy().view(np.uint32)[0],
            int(ws[N.WORKSPACE_BYTES - 1152:].count_nonzero().item()))


def test_noalloc_amax_two_calls_second_smaller():
    big = synth.make("activation")["x"]  # 8192 x 4096, Student-t with x50 channels
    xb = torch.from_numpy(big.view(np.int16)).view(torch.bfloat16).cuda()
    rng = np.random.default_rng(7)
    small = synth.to_bf16_bits((rng.standard_normal(300 * 1024 + 24) * 0.01).astype(np.float32))
    small[12345] = 0x4480  # 1024.0, the maximum of the small tensor
    xs = torch.from_numpy(small.view(np.int16)).view(torch.bfloat16).cuda()
    for what, x in (("8192x4096", xb), ("307224 elements", xs)):
        ref, got, dirty = _amax_both(x)
        assert got == ref, (what, hex(got), hex(ref))
        assert dirty == 0, "the workspace's counters are left zero"
    assert np.frombuffer(np.uint32(_amax_both(xs)[1]).tobytes(), np.float32)[0] == 1024.0


def test_noalloc_amax_rejects_before_launch():
    lib = N.lib()
    assert lib.nvfp4_tensor_amax_noalloc(None, 16, 0x100000, None) == N.ERR_INVALID
    assert lib.nvfp4_tensor_amax_noalloc(0x100000, -1, 0x100000, None) == N.ERR_INVALID
    assert lib.nvfp4_tensor_amax_noalloc(0x100004, 16, 0x100000, None) == N.ERR_INVALID
    assert lib.nvfp4_tensor_amax_noalloc(0x100000, 16, None, None) == N.ERR_INVALID
