"""Shared helpers for the GPU tests: moving bf16 bit patterns to the device,
oracle-derived code boundaries, and tolerance checks."""
import sys

import numpy as np

import oracle as O


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def dev_f32(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def f32_of_bits(p):
    return np.array([p], np.uint32).view(np.float32)[0]


def boundaries(code_of_pattern, top_pattern, ncodes):
    """Smallest non-negative binary32 bit pattern at which a monotone encoder
    (pattern -> code in 0..ncodes-1) first reaches code k, for k = 1..ncodes-1,
    found by bisection on the oracle."""
    out = []
    lo_start = 0
    for k in range(1, ncodes):
        lo, hi = lo_start, top_pattern
        if code_of_pattern(hi) < k:
            out.append(None)
            continue
        while lo < hi:
            mid = (lo + hi) // 2
            if code_of_pattern(mid) >= k:
                hi = mid
            else:
                lo = mid + 1
        out.append(lo)
        lo_start = lo
    return out


def segments(lo, hi, bounds, limit):
    """Split the pattern range [lo, hi) into runs of constant code given the
    start patterns `bounds` of codes 1.. (None = never reached); patterns at
    or above `limit` are left out.  Yields (start, end, code)."""
    edges = [(0, 0)] + [(b, k) for k, b in enumerate(bounds, start=1) if b is not None]
    for j, (start, k) in enumerate(edges):
        end = edges[j + 1][0] if j + 1 < len(edges) else limit
        a, b = max(start, lo), min(end, hi, limit)
        if a < b:
            yield a, b, k


def assert_close_rel(got, ref, rel=1e-5, what="values"):
    """|got - ref| <= rel * |ref| elementwise; exact where ref == 0; NaN where
    ref is NaN."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), f"{what}: NaN positions differ"
    g, r = got[~nan], ref[~nan]
    err = np.abs(g - r)
    ok = err <= rel * np.abs(r)
    if not ok.all():
        i = int(np.argmax(~ok))
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} beyond rel {rel}; "
                             f"first at {i}: got {g[i]!r} ref {r[i]!r}")
    return float((err / np.where(r == 0, 1, np.abs(r))).max()) if err.size else 0.0
