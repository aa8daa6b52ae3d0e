"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and rounds them to bf16; it holds none of the
quantization or GEMM arithmetic, so the GPU path and the CPU oracle can both be fed from it
without sharing any of the method.

Recipe: values are drawn in fp32 from NumPy's PCG64, seeded by a SeedSequence built from a
base seed and a stable hash of the tensor's name, then rounded to bf16 (round to nearest even,
PyTorch's CPU cast).  No dataset or trained weights are used anywhere.
"""
from __future__ import annotations

import zlib

import numpy as np
import torch


def rng(seed: int, name: str) -> np.random.Generator:
    """Independent stream for (seed, tensor name)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, zlib.crc32(name.encode())])))


def to_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def normal(shape, std: float, seed: int, name: str) -> torch.Tensor:
    """N(0, std^2) (std is the standard deviation), rounded to bf16."""
    g = rng(seed, name)
    return to_bf16(g.standard_normal(size=shape, dtype=np.float32) * np.float32(std))


def activations_with_outliers(m: int, k: int, seed: int, name: str, frac: float = 0.01,
                              factor: float = 50.0) -> torch.Tensor:
    """N(0,1) activations [m, k] where round(frac*k) channels (columns, chosen without
    replacement, the same for every row) are multiplied by ``factor``."""
    g = rng(seed, name)
    x = g.standard_normal(size=(m, k), dtype=np.float32)
    n_out = int(round(frac * k))
    cols = g.choice(k, size=n_out, replace=False)
    x[:, cols] *= np.float32(factor)
    return to_bf16(x)


def student_t(shape, nu: float, seed: int, name: str) -> torch.Tensor:
    """Unscaled Student-t(nu) values, rounded to bf16."""
    g = rng(seed, name)
    return to_bf16(g.standard_t(nu, size=shape).astype(np.float32))


def moe_routing(tokens: int, experts: int, topk: int, alpha: float, seed: int,
                name: str = "moe/routing") -> np.ndarray:
    """Rows per expert after top-k routing with Zipf(alpha)-skewed expert popularity.

    Each token picks ``topk`` distinct experts by the Gumbel-top-k trick on log p_e with
    p_e proportional to (e+1)^-alpha (the same law as sampling without replacement).  Returns
    int64 counts per expert; their sum is tokens * topk.
    """
    g = rng(seed, name)
    logp = -alpha * np.log(np.arange(1, experts + 1, dtype=np.float64))
    counts = np.zeros(experts, dtype=np.int64)
    step = 4096
    for t0 in range(0, tokens, step):
        n = min(step, tokens - t0)
        gumbel = -np.log(-np.log(g.random(size=(n, experts))))
        top = np.argpartition(-(logp[None, :] + gumbel), topk - 1, axis=1)[:, :topk]
        counts += np.bincount(top.reshape(-1), minlength=experts)
    return counts


def offsets_from_counts(counts) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(counts, dtype=np.int64))]).astype(np.int64)


def random_bf16_bits(shape, seed: int, name: str) -> np.ndarray:
    """Uniformly random bf16 bit patterns (every class: zeros, subnormals, inf, NaN)."""
    g = rng(seed, name)
    return g.integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)
