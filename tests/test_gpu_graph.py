"""HIP graph capture of the launch-bound 256x1024 step: tensor amax, 4/6
quantize with the 4/6 count, max->6 quantize and dequantize, captured once
from prepared launches and replayed several times on alternating inputs.
Between replays the program does its own eager work (copying the next input
in, reading the results back, synchronizing); every replay must equal the
eager launches on the same input, and the oracle.  The count is cleared
inside the graph by a fill kernel (no memset node)."""
import numpy as np
import pytest

import oracle as O
from helpers import dev_bf16, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
nv = pytest.importorskip("nvfp4_block_scaled_02_amd")
from nvfp4_block_scaled_02_amd import synth  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def test_graph_replays_match_eager_and_oracle():
    rows, cols = 256, 1024
    inputs = [synth.make("weight-1k")["x"],
              synth.random_bf16(rows, cols, seed=11, scale=3.0, outlier_frac=0.002, outlier_mult=40.0)]
    dev = torch.device("cuda:0")
    x = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)
    amax = torch.empty(1, dtype=torch.float32, device=dev)
    ws = nv.workspace(dev)
    o46 = {"codes": torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev),
           "scales": torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev),
           "count4": torch.zeros(1, dtype=torch.int64, device=dev)}
    o6 = {"codes": torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev),
          "scales": torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)}
    xh = torch.empty((rows, cols), dtype=torch.float32, device=dev)
    gm = 448.0
    launches = [nv.prepare_tensor_amax(x, amax, workspace=ws),
                nv.prepare_quantize(x, amax, select="4over6", global_max=gm, out=o46, workspace=ws)[0],
                nv.prepare_quantize(x, amax, select="6", global_max=gm, out=o6)[0],
                nv.prepare_dequantize(o46["codes"], o46["scales"], amax, global_max=gm, out=xh)[0]]

    def step():
        o46["count4"].zero_()
        for f in launches:
            f()

    def snapshot():
        torch.cuda.synchronize()
        return {"amax": amax.item(), "codes": o46["codes"].cpu().numpy(),
                "scales": o46["scales"].cpu().numpy(), "count4": int(o46["count4"].item()),
                "codes6": o6["codes"].cpu().numpy(), "scales6": o6["scales"].cpu().numpy(),
                "xh": xh.cpu().numpy()}

    # eager reference per input
    eager = []
    for xb in inputs:
        x.copy_(dev_bf16(xb))
        step()
        eager.append(snapshot())
    # the oracle agrees with the eager launches
    for xb, e in zip(inputs, eager):
        A = float(O.tensor_amax(xb))
        assert e["amax"] == A
        c, s, n4 = O.quantize(xb, A, select=O.SELECT_4OVER6, global_max=gm)
        assert np.array_equal(e["codes"], c) and np.array_equal(e["scales"], s) and e["count4"] == n4
        c6, s6, _ = O.quantize(xb, A, select=O.SELECT_6, global_max=gm)
        assert np.array_equal(e["codes6"], c6) and np.array_equal(e["scales6"], s6)
        assert np.array_equal(e["xh"], O.dequantize(c, s, A, select=O.SELECT_4OVER6, global_max=gm))

    g = torch.cuda.CUDAGraph()
    x.copy_(dev_bf16(inputs[0]))
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(6):
        k = r % 2
        x.copy_(dev_bf16(inputs[k]))      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        log(f"graph replay {r} on input {k}: count4 {got['count4']}")
        for key, ref in eager[k].items():
            if isinstance(ref, np.ndarray):
                assert np.array_equal(got[key], ref), (r, key)
            else:
                assert got[key] == ref, (r, key, got[key], ref)
