"""The bench's output contract: one JSON line with the metric, the whole-job
value, the roofline of the metric's kernel and the CPU baseline; one GPU only;
no fallback when the GPU or the HIP library is missing."""
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

CONTRACT_KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                 "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                 "roofline", "cpu_baseline"}
ROOFLINE_KEYS = {"bound", "achieved", "peak", "unit", "frac", "traffic"}


def _run(args, timeout):
    return subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py")] + args,
                          cwd=ROOT, capture_output=True, text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"], 120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_kernel_entry_and_roofline_arithmetic():
    n = 8192 * 4096
    e = bench.kernel_entry(15.0, n, bench.B_QUANT)
    gbps = n * 2.5625 / 15e-6 / 1e9
    assert abs(e["gbps"] - gbps) <= 0.05
    assert abs(e["frac_hbm"] - gbps / 8000.0) <= 5e-5
    assert abs(e["gelem_per_s"] - n / 15e-6 / 1e9) <= 0.05
    kernels = {"quantize_4over6": e, "dequantize_f32_mse": bench.kernel_entry(40.0, n, bench.B_DEQ_MSE)}
    line = bench.finish({}, kernels, None, {"quantize_4over6": 86_000_000},
                        roofline_kernel="quantize_4over6")
    rl = line["roofline"]
    assert ROOFLINE_KEYS <= set(rl)
    assert rl["kernel"] == "quantize_4over6" and rl["bound"] == "hbm" and rl["unit"] == "GB/s"
    assert rl["achieved"] == e["gbps"] and rl["peak"] == 8000.0 and rl["frac"] == e["frac_hbm"]
    assert rl["traffic"] == 86_000_000
    # without a named kernel the longest one is the roofline's
    assert bench.finish({}, dict(kernels), None)["roofline"]["kernel"] == "dequantize_f32_mse"


def test_committed_counters_need_matching_sources(tmp_path, monkeypatch):
    """A workload's committed PMC figures feed traffic and the VALU ceiling
    only while the hash of the kernel's sources matches."""
    n = 8192 * 4096
    key = "quantize_4over6"
    entry = {"bytes_per_launch": 86_100_000, "valu_busy_pct": 50.0, "valu_instr_per_block": 200.0,
             "source_sha256": bench.source_hash(bench.kernel_sources(key))}
    (tmp_path / "activation_8192x4096_step_counters.json").write_text(
        json.dumps({"kernels": {key: entry}}))
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    args = SimpleNamespace(workload="activation")
    line = bench.finish({}, {key: bench.kernel_entry(16.0, n, bench.B_QUANT)}, args, None, key)
    assert line["roofline"]["traffic"] == 86_100_000
    assert line["kernels"][key]["valu_busy_pct"] == 50.0
    assert line["valu"]["issue_bound_us"] == 8.0 and line["valu"]["busy_pct"] == 50.0
    entry["source_sha256"] = "0" * 64  # taken on other sources: not reported
    (tmp_path / "activation_8192x4096_step_counters.json").write_text(
        json.dumps({"kernels": {key: entry}}))
    line = bench.finish({}, {key: bench.kernel_entry(16.0, n, bench.B_QUANT)}, args, None, key)
    assert line["roofline"]["traffic"] is None and "valu" not in line


def test_committed_counters_match_the_current_sources():
    """Every committed counters file names each kernel's sources as the bench
    does (so a change to a kernel voids exactly its own figures)."""
    for name in bench.PROFILE_NAMES.values():
        path = os.path.join(bench.PROFILE_DIR, name + "_counters.json")
        if not os.path.exists(path):
            continue
        with open(path) as f:
            kernels = json.load(f)["kernels"]
        for key, t in kernels.items():
            assert t["sources"] == bench.kernel_sources(key), (name, key)


def test_base_line_fields():
    args = SimpleNamespace(steps=7, warmup=3)
    line = bench.base_line(bench.METRIC, 1234.56, "GB/s", args, 0.07, "w", {"rows": 2}, 1000)
    assert line["metric"] == bench.METRIC and line["value"] == 1234.6 and line["n_gpus"] == 1
    assert line["steps"] == 7 and line["warmup"] == 3 and line["higher_is_better"] is True
    assert line["config"] == {"workload": "w", "rows": 2} and line["data"] == "synthetic"


def test_no_gpu_fails_loudly():
    """Without a GPU the bench stops with an error and prints no line."""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _run(["--steps", "1", "--warmup", "0", "--no-cpu-baseline"], 300)
    assert r.returncode != 0
    assert not any(l.startswith("{") for l in r.stdout.splitlines())


@pytest.mark.gpu
def test_default_line_on_the_gpu():
    """A short default run prints exactly one line with every contract field,
    consistent with itself."""
    r = _run(["--steps", "10", "--warmup", "5", "--no-cpu-baseline"], 300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert CONTRACT_KEYS <= set(d)
    assert d["metric"] == bench.METRIC and d["unit"] == "GB/s" and d["n_gpus"] == 1
    assert d["steps"] == 10 and d["warmup"] == 5 and d["config"]["workload"]
    rl = d["roofline"]
    assert ROOFLINE_KEYS <= set(rl) and rl["kernel"] == "quantize_4over6"
    assert d["value"] == rl["achieved"] == d["kernels"]["quantize_4over6"]["gbps"]
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) <= 1e-4
    assert 0.0 < rl["frac"] < 1.0
    # the value is the metric's kernel: 2.5625 bytes per element over its time
    k = d["kernels"]["quantize_4over6"]
    expect = 8192 * 4096 * 2.5625 / (k["us"] * 1e-6) / 1e9
    assert abs(k["gbps"] - expect) <= 1e-3 * expect
    assert d["cpu_baseline"] is None
