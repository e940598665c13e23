"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and stores them in the input dtypes; it
holds none of the quantize / fold / GEMM arithmetic, so both the HIP path and
the CPU oracle can take their inputs from here without sharing any of the
method.  Every stream is keyed by a tuple (config id, tensor id, step, ...)
through numpy's PCG64 seeding, so any one tensor can be regenerated alone.
"""
from __future__ import annotations

import numpy as np

# tensor ids used in the keys
T_X, T_W, T_BIAS, T_DY, T_ASCALE, T_BSCALE, T_QUANT = 0, 1, 2, 3, 4, 5, 6


def rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def gaussian_f32(shape, sigma: float, *key: int) -> np.ndarray:
    """fp32 samples of N(0, sigma^2)."""
    g = rng(*key)
    return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Store fp32 samples as bf16 (round to nearest even, via torch's CPU cast);
    returns the uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def gaussian(shape, sigma: float, dtype: str, *key: int) -> np.ndarray:
    """N(0, sigma^2) samples in storage form: uint16 bits for 'bf16',
    np.float16 for 'f16', np.float32 for 'f32'."""
    x = gaussian_f32(shape, sigma, *key)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


def loguniform_scale(lo_log2: float, hi_log2: float, *key: int) -> np.float32:
    """One fp32 scale 2^U(lo, hi)."""
    u = rng(*key).uniform(lo_log2, hi_log2)
    return np.float32(2.0 ** u)


def random_bits_f32(n: int, *key: int) -> np.ndarray:
    """n uniformly random fp32 bit patterns (every class: NaN, inf, subnormal)."""
    return rng(*key).integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32).view(np.float32)


def to_torch(x: np.ndarray, dtype: str):
    """CPU torch tensor of the storage array (bf16 bits are reinterpreted)."""
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x))


def device_gaussian(shape, sigma: float, dtype, seed: int, device="cuda"):
    """N(0, sigma^2) drawn on the device with a seeded torch generator (for
    large benchmark inputs where host generation would dominate)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * sigma).to(dtype)
