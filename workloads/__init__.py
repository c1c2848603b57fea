"""Seeded synthetic inputs for the micro-scaled FP4 hot path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no scale rule, no rounding to FP4/FP8, no transform).  Both
the CPU oracle's tests and the GPU library's tests and benchmark take their
inputs from here, so the two sides see identical bytes.

Shapes and value distributions follow the workloads described for the method:
N(0,1) activations with a few outlier channels scaled by tens of times
("NVIDIA NVFP4 与 Micro-Scaling" page, section 四, outlier channels), and
small-magnitude weights.  The pages' own models and datasets are not available,
so these seeded tensors stand in for them.

Every generator returns numpy arrays.  bf16 tensors are returned as their raw
16-bit patterns (numpy uint16), produced by torch's round-to-nearest-even cast
of the float32 draw; the cast is input preparation, not part of the method.
"""
from __future__ import annotations

import numpy as np

SEED_TINY = 1001
SEED_ACTIVATION = 1002
SEED_GEMV = 1003
SEED_GEMM = 1004
SEED_ROTATE = 1005
SEED_SR = 0x5EED


def _rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), via torch's RNE cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal(shape, seed: int, std: float = 1.0) -> np.ndarray:
    a = _rng(seed).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def with_outlier_channels(a: np.ndarray, n_channels: int, factor: float, seed: int) -> np.ndarray:
    """Scale n_channels whole columns (channels) of a 2-D array by factor."""
    if n_channels <= 0:
        return a
    cols = a.shape[-1]
    ch = _rng(seed ^ 0xC0FFEE).choice(cols, size=min(n_channels, cols), replace=False)
    a[..., ch] *= np.float32(factor)
    return a


def with_outlier_entries(a: np.ndarray, frac: float, factor: float, rng: np.random.Generator) -> np.ndarray:
    """Scale a fraction of individual entries (chosen over the flat index) by factor."""
    n = int(round(a.size * frac))
    idx = rng.choice(a.size, size=n, replace=False)
    flat = a.reshape(-1)
    flat[idx] *= np.float32(factor)
    return a


# ---------------------------------------------------------------- workloads
def tiny_pair(rows: int = 64, cols: int = 256, seed: int = SEED_TINY):
    """Tiny NVFP4/MXFP4 reference case: A and W fp32 [rows, cols] ~ N(0,1),
    1% of the entries of each multiplied by 50."""
    rng = _rng(seed)
    A = rng.standard_normal((rows, cols), dtype=np.float32)
    W = rng.standard_normal((rows, cols), dtype=np.float32)
    with_outlier_entries(A, 0.01, 50.0, rng)
    with_outlier_entries(W, 0.01, 50.0, rng)
    return A, W


def activation(rows: int = 8192, cols: int = 8192, n_outlier: int = 8, factor: float = 40.0,
               seed: int = SEED_ACTIVATION, as_bf16: bool = True):
    """Activation tensor ~ N(0,1) with n_outlier channels scaled by factor."""
    a = normal((rows, cols), seed)
    with_outlier_channels(a, n_outlier, factor, seed)
    return f32_to_bf16_bits(a) if as_bf16 else a


def gemv_weight(n: int = 27648, k: int = 5120, seed: int = SEED_GEMV):
    """Decode GEMV weight W [n, k] ~ N(0, 0.02^2) as bf16 bits."""
    return f32_to_bf16_bits(normal((n, k), seed, std=0.02))


def gemv_x(batch: int, k: int = 5120, seed: int = SEED_GEMV):
    """Decode GEMV activations x [batch, k] ~ N(0,1) as bf16 bits."""
    return f32_to_bf16_bits(normal((batch, k), seed + 7919 * (batch + 1)))


def gemm_a(m: int = 8192, k: int = 8192, outlier_frac: float = 0.005, factor: float = 40.0,
           seed: int = SEED_GEMM):
    """Prefill GEMM activations A [m, k] ~ N(0,1) with round(outlier_frac*k)
    outlier channels scaled by factor, as bf16 bits."""
    a = normal((m, k), seed)
    with_outlier_channels(a, max(1, int(round(outlier_frac * k))), factor, seed)
    return f32_to_bf16_bits(a)


def gemm_w(n: int = 28672, k: int = 8192, seed: int = SEED_GEMM):
    """Prefill GEMM weights W [n, k] ~ N(0, 0.02^2) as bf16 bits."""
    return f32_to_bf16_bits(normal((n, k), seed + 1, std=0.02))


def rotate_input(rows: int = 16384, cols: int = 8192, n_outlier: int = 16, factor: float = 60.0,
                 seed: int = SEED_ROTATE):
    """Rotate-then-quantize activations ~ N(0,1) with n_outlier channels x factor, bf16 bits."""
    a = normal((rows, cols), seed)
    with_outlier_channels(a, n_outlier, factor, seed)
    return f32_to_bf16_bits(a)


SEED_MOE = 1006


def moe_group_sizes(num_experts: int = 64, rows: int = 32768, seed: int = SEED_MOE) -> list:
    """Rows routed to each expert of an MoE layer (tokens x top-k assignments):
    a multinomial draw of `rows` over expert popularities exp(N(0, 0.5^2)), so
    the loads are uneven and some experts may get none.  Sums to rows."""
    rng = _rng(seed)
    p = np.exp(rng.normal(0.0, 0.5, num_experts))
    return [int(c) for c in rng.multinomial(rows, p / p.sum())]


def random_codes(shape, seed: int) -> np.ndarray:
    """Uniform random 4-bit codes packed two per byte (any byte value is valid)."""
    return _rng(seed).integers(0, 256, size=shape, dtype=np.uint8)


def random_bytes(shape, lo: int, hi: int, seed: int) -> np.ndarray:
    """Uniform random bytes in [lo, hi] (for block-scale bytes in a chosen range)."""
    return _rng(seed).integers(lo, hi + 1, size=shape, dtype=np.uint8)
