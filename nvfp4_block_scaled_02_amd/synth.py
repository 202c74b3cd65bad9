"""Seeded synthetic inputs shaped like the pages' workloads.

This module draws random numbers and nothing else: it holds none of the
quantization arithmetic, and both the GPU tests and the CPU oracle consume the
same arrays it returns (bf16 bit patterns as uint16, fp32 as float32).

Recipe (numpy Generator(PCG64(seed)); draws in float64, cast to float32, then
to bfloat16 with round-to-nearest-even through torch):
  weight-1k   256 x 1024  N(0,1); round(0.001 N) distinct positions x 20  (seed 0)
  weight      4096 x 4096 N(0,0.02) x per-row lognormal(0, 0.5)           (seed 1)
  activation  8192 x 4096 Student-t(3) x 0.5; 8 fixed channels x 50       (seed 2)
  qat         W 14336 x 4096 N(0,0.02) bf16; G N(0,1e-3) float32          (seed 3)
  gradient    16384 x 8192 N(0,1) x per-row 10^U(-3,0)                    (seed 4)
  heavy       4096 x 4096  N(0,1) x per-element U(1,9): the heavy-tailed
              activation stand-in of the "UE5M3" blog's scale-format
              experiment (实验)                                          (seed 5)
  wide        4096 x 4096  N(0,1) x 2^(-24 U(0,1)) per 16-element block: block
              magnitudes spanning 24 binades, wider than the E4M3 block-scale
              range under a per-tensor outer scale (about 17.8 binades)  (seed 6)
`rows` gives a smaller instance of the same recipe (per-row factors, outlier
channels and outlier positions are drawn at the full shape first, so the kept
rows see the same ones).  No public dataset
or model file is used; these tensors stand in for LLM weights, S = 8192
training-length activations, a Llama-class MLP weight and its gradient, and
backward-pass gradients.
"""
import numpy as np
import torch

SHAPES = {
    "weight-1k": (256, 1024),
    "weight": (4096, 4096),
    "activation": (8192, 4096),
    "qat": (14336, 4096),
    "gradient": (16384, 8192),
    "heavy": (4096, 4096),
    "wide": (4096, 4096),
}
SEEDS = {"weight-1k": 0, "weight": 1, "activation": 2, "qat": 3, "gradient": 4, "heavy": 5,
         "wide": 6}


def to_bf16_bits(a) -> np.ndarray:
    """float64/float32 array -> bfloat16 bit patterns (uint16), RNE via torch."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make(name: str, rows: int = None):
    """Returns a dict with 'x' (bf16 bits, [rows, cols]) and, for 'qat', 'g'
    (float32 upstream gradient)."""
    R, C = SHAPES[name]
    r = R if rows is None else int(rows)
    rng = np.random.Generator(np.random.PCG64(SEEDS[name]))
    if name == "weight-1k":
        x = rng.standard_normal((R, C))
        n_out = int(round(0.001 * R * C))
        idx = rng.choice(R * C, n_out, replace=False)
        x.reshape(-1)[idx] *= 20.0
        x = x[:r]
    elif name == "weight":
        f = rng.lognormal(0.0, 0.5, size=R)
        x = rng.standard_normal((r, C)) * 0.02 * f[:r, None]
    elif name == "activation":
        ch = np.sort(rng.choice(C, 8, replace=False))
        x = rng.standard_t(3, size=(r, C)) * 0.5
        x[:, ch] *= 50.0
    elif name == "qat":
        x = rng.standard_normal((r, C)) * 0.02
        g = rng.standard_normal((r, C)) * 1e-3
        return {"x": to_bf16_bits(x), "g": g.astype(np.float32)}
    elif name == "gradient":
        f = 10.0 ** rng.uniform(-3.0, 0.0, size=R)
        x = rng.standard_normal((r, C)) * f[:r, None]
    elif name == "heavy":
        x = rng.standard_normal((r, C)) * rng.uniform(1.0, 9.0, size=(r, C))
    elif name == "wide":
        f = 2.0 ** (-24.0 * rng.uniform(0.0, 1.0, size=(R, C // 16)))
        x = (rng.standard_normal((r, C // 16, 16)) * f[:r, :, None]).reshape(r, C)
    else:
        raise KeyError(name)
    return {"x": to_bf16_bits(x)}


def random_bf16(rows: int, cols: int, seed: int, scale: float = 1.0, outlier_frac: float = 0.0,
                outlier_mult: float = 1.0) -> np.ndarray:
    """Generic seeded bf16 matrix for edge-case tests."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((rows, cols)) * scale
    if outlier_frac > 0:
        x[rng.random((rows, cols)) < outlier_frac] *= outlier_mult
    return to_bf16_bits(x)
