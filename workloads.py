"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no quantizer arithmetic: it only draws numbers and casts them to bf16.
Every tensor is drawn as float64 with numpy's PCG64 ``default_rng(seed)``, cast to float32,
then to bfloat16 by torch's CPU cast (round to nearest even).

The pages measure on model gradients and activations (Llama-3.2-1B block 0 in the
unbiasedness figure of the Quartet II summary; Llama-2 / Nanochat training runs in the
"Experiments" section of the Telegram digest), none of which is available here; these
distributions stand in for them:

* ``c1``  256 x 1024, i.i.d. N(0, 1)                                   (seed 0)
* ``c2``  4096 x 4096 weight-like: Student-t(3) * 0.02, then 0.1% of the entries
          (16777, without replacement) multiplied by 50                 (seed 0)
* ``c3``  16384 x 2048 grad-output: per-row magnitude 10**U(-6, 1) times N(0, 1)  (seed 0)
* ``c4``  16384 x 8192 activation / gradient: N(0, 1) times a per-column log-normal(0, 1)
          scale                                                          (seed 0)
* ``c4w`` 8192 x 8192 second GEMM operand, 0.02 * N(0, 1)               (seed 1)
"""
from __future__ import annotations

import numpy as np
import torch

SHAPES = {
    "c1": (256, 1024),
    "c2": (4096, 4096),
    "c3": (16384, 2048),
    "c4": (16384, 8192),
    "c4w": (8192, 8192),
}


def to_bf16(x64: np.ndarray) -> torch.Tensor:
    """float64 -> float32 -> bfloat16 (CPU tensor, contiguous)."""
    return torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32)).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The uint16 bit patterns of a CPU bfloat16 tensor (no copy of values)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def c1(seed: int = 0) -> torch.Tensor:
    return to_bf16(np.random.default_rng(seed).standard_normal(SHAPES["c1"]))


def c2(seed: int = 0, shape=None) -> torch.Tensor:
    shape = shape or SHAPES["c2"]
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, shape) * 0.02
    n = x.size
    k = max(1, n // 1000) if shape != SHAPES["c2"] else 16777
    idx = rng.choice(n, k, replace=False)
    x.flat[idx] *= 50.0
    return to_bf16(x)


def c3(seed: int = 0, shape=None) -> torch.Tensor:
    shape = shape or SHAPES["c3"]
    rng = np.random.default_rng(seed)
    m = 10.0 ** rng.uniform(-6.0, 1.0, (shape[0], 1))
    return to_bf16(m * rng.standard_normal(shape))


def c4(seed: int = 0, shape=None) -> torch.Tensor:
    shape = shape or SHAPES["c4"]
    rng = np.random.default_rng(seed)
    cs = rng.lognormal(0.0, 1.0, shape[1])
    return to_bf16(rng.standard_normal(shape) * cs)


def c4w(seed: int = 1, shape=None) -> torch.Tensor:
    shape = shape or SHAPES["c4w"]
    return to_bf16(0.02 * np.random.default_rng(seed).standard_normal(shape))


def normal(shape, seed: int = 0, scale: float = 1.0) -> torch.Tensor:
    return to_bf16(scale * np.random.default_rng(seed).standard_normal(shape))


GENERATORS = {"c1": c1, "c2": c2, "c3": c3, "c4": c4, "c4w": c4w}
