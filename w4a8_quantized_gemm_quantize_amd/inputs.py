"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the quantization method: it only draws
random numbers and rounds them to bf16 once, so that the same bf16 bit
patterns can be handed to the HIP library and to the CPU oracle.

Generator: numpy ``Generator(PCG64(SeedSequence([seed, stream])))`` with
stream 0 = activations, 1 = weights, 2 = outlier positions.  Values are drawn
in float32 and rounded to bf16 (round to nearest, ties to even); that bf16
tensor is the canonical input.
"""
from __future__ import annotations

import numpy as np

STREAM_A = 0
STREAM_W = 1
STREAM_OUTLIERS = 2


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even. Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lower = u & 0xFFFF
    upper = u >> 16
    round_up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    return (upper + round_up.astype(np.uint64)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def activations(m: int, k: int, seed: int = 0, dist: str = "normal",
                outlier_frac: float = 0.0, outlier_mult: float = 20.0) -> np.ndarray:
    """bf16 bits [m, k].

    dist: "normal" (N(0,1)) or "student_t" (unit-scale Student t, 3 degrees of
    freedom).  outlier_frac > 0 multiplies exactly round(frac * m * k) distinct
    positions (drawn without replacement from the outlier stream) by
    outlier_mult before the bf16 rounding.
    """
    g = rng(seed, STREAM_A)
    if dist == "normal":
        x = g.standard_normal((m, k), dtype=np.float32)
    elif dist == "student_t":
        x = g.standard_t(3, size=(m, k)).astype(np.float32)
    else:
        raise ValueError(dist)
    if outlier_frac > 0 and m * k > 0:
        count = int(round(outlier_frac * m * k))
        pos = rng(seed, STREAM_OUTLIERS).choice(m * k, size=count, replace=False)
        flat = x.reshape(-1)
        flat[pos] *= np.float32(outlier_mult)
    return f32_to_bf16_bits(x)


def weights(n: int, k: int, seed: int = 0, sigma: float = 0.02) -> np.ndarray:
    """bf16 bits [n, k] drawn from N(0, sigma^2) (nn.Linear layout: out x in)."""
    g = rng(seed, STREAM_W)
    w = g.standard_normal((n, k), dtype=np.float32) * np.float32(sigma)
    return f32_to_bf16_bits(w)


# Workloads: shapes and value distributions of the measured configurations.
WORKLOADS = {
    "tiny": dict(m=16, k=256, n=256, dist="normal", outlier_frac=0.0, out="f32"),
    "decode": dict(m=8, k=4096, n=4096, dist="normal", outlier_frac=0.001, out="bf16"),
    "prefill": dict(m=4096, k=4096, n=14336, dist="normal", outlier_frac=0.001, out="bf16"),
    "ffn_down_m1": dict(m=1, k=28672, n=8192, dist="student_t", outlier_frac=0.0, out="bf16"),
    "ffn_down_m64": dict(m=64, k=28672, n=8192, dist="student_t", outlier_frac=0.0, out="bf16"),
    "ffn_down_m2048": dict(m=2048, k=28672, n=8192, dist="student_t", outlier_frac=0.0,
                           out="bf16"),
}

# Standalone quantizer workload: 64M bf16 elements, N(0,1), as [65536, 1024].
QUANTIZER = dict(rows=65536, cols=1024, blocks=(32, 128))


def workload_inputs(name: str, seed: int = 0):
    """-> (a_bf16 [m,k], w_bf16 [n,k], spec) for a named GEMM workload."""
    spec = WORKLOADS[name]
    a = activations(spec["m"], spec["k"], seed, spec["dist"], spec["outlier_frac"])
    w = weights(spec["n"], spec["k"], seed)
    return a, w, spec
