"""Seeded tensor generation.

Each layer draws from ``numpy.random.default_rng(seed)`` (PCG64): the input x
first, then the filter w, both in float64, cast to float32. For the half
precision variants the *same* float32 draws are rounded once, to nearest-even,
to float16 or bfloat16; the oracle and the GPU then read identical bits.
"""
from __future__ import annotations

import math

import numpy as np
import torch

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _draw(rng: np.random.Generator, shape, dist: str, fan_in: int) -> np.ndarray:
    if dist == "normal":
        a = rng.standard_normal(shape)
    elif dist == "uniform":
        a = rng.uniform(-1.0, 1.0, shape)
    elif dist == "he":
        a = rng.standard_normal(shape) * math.sqrt(2.0 / fan_in)
    elif dist == "int3":
        # small integers in [-3, 3]: every product and partial sum is exact
        a = rng.integers(-3, 4, shape).astype(np.float64)
    elif dist == "ones":
        a = np.ones(shape)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return a.astype(np.float32)


def round_to_dtype(a32: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 array -> CPU tensor of the storage dtype (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(TORCH_DTYPES[dtype]).contiguous()


def make_tensor(shape, dist: str, seed: int, dtype: str = "f32", fan_in: int = 1) -> torch.Tensor:
    rng = np.random.default_rng(seed)
    return round_to_dtype(_draw(rng, shape, dist, fan_in), dtype)


def make_inputs(N, Cin, H, W, Cout, KH, KW, seed, dtype="f32",
                x_dist="normal", w_dist="he"):
    """Return (x, w) as contiguous CPU tensors of ``dtype`` (x drawn first, then w)."""
    rng = np.random.default_rng(seed)
    x = _draw(rng, (N, Cin, H, W), x_dist, Cin * KH * KW)
    w = _draw(rng, (Cout, Cin, KH, KW), w_dist, Cin * KH * KW)
    return round_to_dtype(x, dtype), round_to_dtype(w, dtype)


def make_config_inputs(cfg, dtype):
    return make_inputs(cfg.N, cfg.Cin, cfg.H, cfg.W, cfg.Cout, cfg.KH, cfg.KW,
                       cfg.seed, dtype, cfg.x_dist, cfg.w_dist)
