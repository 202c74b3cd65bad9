"""Benchmark: NVFP4 Four-Over-Six quantization of an 8192 x 4096 bf16
activation tensor on one MI355X.

One step is the whole hot path of that workload: tensor amax (current
scaling) -> Four-Over-Six quantize along the hidden dimension (E4M3 scales,
outer scale from FP8 max 256) -> dequantize to binary32 with the binary64
squared-error report (per-tensor MSE).  Inputs are resident in HBM before the
timed region.  Eight buffer sets (8 x 64 MiB of input, more than the 256 MB
Infinity Cache) are used in rotation so each launch streams from HBM.

Prints one JSON line.  `value` is the step's algorithmic bytes per second
(GB/s); per-kernel figures sit under "kernels", the dominant kernel's under
"roofline", and the CPU oracle timed on a sample under "cpu_baseline".
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
WORKLOAD = "activation"
N_SETS = 8
PROFILE_DIR = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILE_DIR, "quantize_4over6_activation_8192x4096_traffic.json")
KERNEL_SOURCES = ["quantize.hip", "device.hpp", "common.hpp"]

# algorithmic bytes per element (read + written, each byte counted once)
BYTES = {
    "tensor_amax": 2.0,                      # bf16 read
    "quantize_4over6": 2.0 + 0.5 + 1 / 16,   # bf16 read, 4-bit codes + 1 scale byte per 16
    "dequantize_f32_mse": 0.5 + 1 / 16 + 2.0 + 4.0,  # codes+scales+bf16 read, f32 written
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "nvfp4_block_scaled_02_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per quantize launch from the committed PMC summary, if it
    was taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(xb, target_cpu_s=12.0):
    """The oracle, untuned, on the host: the same step on a bounded sample of
    whole rows of the same tensor, repeated until ~target_cpu_s of CPU time."""
    import numpy as np
    import oracle as O

    threads = O.num_threads()
    rows = xb.shape[0]
    sample_rows = rows  # the whole tensor is a bounded sample here (seconds)
    x = xb[:sample_rows]
    n = x.size
    reps, t_wall, t_cpu0 = 0, 0.0, time.process_time()
    while True:
        t0 = time.perf_counter()
        a = O.tensor_amax(x)
        codes, scales, _ = O.quantize(x, a, select=O.SELECT_4OVER6)
        xh = O.dequantize(codes, scales, a, select=O.SELECT_4OVER6)
        O.sse(x, xh)
        t_wall += time.perf_counter() - t0
        reps += 1
        if time.process_time() - t_cpu0 >= target_cpu_s or reps >= 20:
            break
    per_step = t_wall / reps
    step_bytes = n * sum(BYTES.values())
    return {
        "value": round(step_bytes / per_step / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{sample_rows}x{x.shape[1]} rows of the same tensor, full step "
                  f"(amax, 4/6 quantize, dequantize, SSE), {reps} reps, "
                  f"{per_step * 1e3:.1f} ms/step wall, {threads} OpenMP threads",
        "gelem_per_s": round(n / per_step / 1e9, 4),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-once", action="store_true",
                    help="run a 256 MiB copy and a few quantize launches for PMC counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by rows with no exchange besides an amax all-reduce; "
              "see the sharding note in the design document).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import nvfp4_block_scaled_02_amd as nv
    from nvfp4_block_scaled_02_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("generating the 8192x4096 activation tensor")
    xb = synth.make(WORKLOAD)["x"]
    rows, cols = xb.shape
    n = rows * cols
    x0 = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
    xs = [x0] + [x0.clone() for _ in range(N_SETS - 1)]
    amaxs = [torch.empty(1, dtype=torch.float32, device=dev) for _ in range(N_SETS)]
    outs = [{"codes": torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev),
             "scales": torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)}
            for _ in range(N_SETS)]
    xh = [torch.empty((rows, cols), dtype=torch.float32, device=dev) for _ in range(N_SETS)]
    gm = nv.default_global_max("e4m3", "4over6")

    if args.profile_once:
        big = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(big)
        dst.copy_(big)
        for i in range(4):
            nv.quantize(xs[i], amaxs[i], select="4over6", out=outs[i])
        torch.cuda.synchronize()
        log("profile-once done: one 256 MiB copy, 4 quantize launches")
        return

    total = args.warmup + args.steps
    sse = torch.zeros(total, dtype=torch.float64, device=dev)

    def step(i):
        k = i % N_SETS
        nv.tensor_amax(xs[k], out=amaxs[k])
        nv.quantize(xs[k], amaxs[k], select="4over6", out=outs[k])
        nv.dequantize(outs[k]["codes"], outs[k]["scales"], amaxs[k], global_max=gm,
                      x_ref=xs[k], sse=sse[i:i + 1], out=xh[k])

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_host0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.warmup, total):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    log(f"timed {args.steps} steps: {ms_step * 1e3:.2f} us/step (host clock {t_host * 1e3 / args.steps:.2f} us/step)")

    # per-kernel average duration: back-to-back launches of one kernel over
    # the rotating buffer sets, bracketed by events on the same stream
    def per_kernel(fn, reps):
        for i in range(N_SETS):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3  # us

    reps = max(args.steps, 40)
    sse_k = torch.zeros(1, dtype=torch.float64, device=dev)
    us = {
        "tensor_amax": per_kernel(lambda i: nv.tensor_amax(xs[i % N_SETS], out=amaxs[i % N_SETS]), reps),
        "quantize_4over6": per_kernel(lambda i: nv.quantize(xs[i % N_SETS], amaxs[i % N_SETS],
                                                            select="4over6", out=outs[i % N_SETS]), reps),
        "dequantize_f32_mse": per_kernel(lambda i: nv.dequantize(
            outs[i % N_SETS]["codes"], outs[i % N_SETS]["scales"], amaxs[i % N_SETS], global_max=gm,
            x_ref=xs[i % N_SETS], sse=sse_k, out=xh[i % N_SETS]), reps),
    }
    kernels = {}
    for k, t in us.items():
        gbps = n * BYTES[k] / (t * 1e-6) / 1e9
        kernels[k] = {"us": round(t, 3), "bytes_per_elem": round(BYTES[k], 4),
                      "gbps": round(gbps, 1), "frac_hbm": round(gbps / HBM_PEAK_GBPS, 4),
                      "gelem_per_s": round(n / (t * 1e-6) / 1e9, 1)}
    dominant = max(us, key=us.get)
    log(f"kernels: {json.dumps(kernels)}")

    # results of the last timed step (report only)
    last = (total - 1) % N_SETS
    mse = float(sse[total - 1].item()) / n
    step_bytes = n * sum(BYTES.values())
    value = step_bytes / (ms_step * 1e-3) / 1e9
    d = kernels[dominant]
    traffic = measured_traffic() if dominant == "quantize_4over6" else None
    line = {
        "metric": "NVFP4 4/6 quantize GB/s (Gelem/s) at 8192x4096 bf16; % of HBM peak",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "activation 8192x4096 bf16 (Student-t(3) x 0.5, 8 channels x 50, seed 2): "
                        "tensor amax -> Four-Over-Six quantize along hidden (E4M3 scales, FP8 max "
                        "256, RNE) -> dequantize to f32 with binary64 MSE report",
            "rows": rows, "cols": cols, "elements": n, "step_bytes": int(step_bytes),
            "buffer_sets": N_SETS,
        },
        "gelem_per_s": round(n / (ms_step * 1e-3) / 1e9, 2),
        "kernels": kernels,
        "roofline": {
            "kernel": dominant,
            "bound": "hbm",
            "achieved": d["gbps"],
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": d["frac_hbm"],
            "traffic": traffic,
        },
        "quantize_roofline": {
            "achieved": kernels["quantize_4over6"]["gbps"], "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": kernels["quantize_4over6"]["frac_hbm"],
            "gelem_per_s": kernels["quantize_4over6"]["gelem_per_s"],
        },
        "mse": mse,
        "amax": float(amaxs[last].item()),
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the host")
        line["cpu_baseline"] = cpu_baseline(xb)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
