"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds input generation only (random draws and their casts to the
storage dtypes) and none of the quantization arithmetic, so that the CPU oracle
and the GPU library can both be fed from it without sharing any of the method.

Recipe (numpy PCG64 via ``default_rng(seed)``): values are
``standard_normal(float32) * sigma + mu``, then one round-to-nearest-even cast
to fp16 (weights) or to fp16/bf16 (activations).  Trained transformer weights
are close to normal, which is the premise behind the NF4 codebook; the layer
shapes below are those of 7B/8B-class decoder layers.
"""

from __future__ import annotations

import numpy as np

NF4, INT4_SYM, INT4_ASYM = 0, 1, 2
F16, BF16 = 0, 1


def normal_f32(shape, seed: int, sigma: float = 1.0, mu: float = 0.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        v *= np.float32(sigma)
    if mu != 0.0:
        v += np.float32(mu)
    return v


def to_f16_bits(v: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(v, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def weight_f16_bits(N: int, K: int, seed: int, sigma: float = 0.02, mu: float = 0.0,
                    outlier_seed: int | None = None, outlier_mult: float = 10.0) -> np.ndarray:
    """fp16 weight bit patterns [N, K] ~ N(mu, sigma^2).  With outlier_seed,
    floor(0.001 * N * K) distinct positions (chosen without replacement) are
    multiplied by outlier_mult in float32 before the single fp16 cast."""
    v = normal_f32((N, K), seed, sigma, mu)
    if outlier_seed is not None:
        n = N * K
        idx = np.random.default_rng(outlier_seed).choice(n, n // 1000, replace=False)
        flat = v.reshape(-1)
        flat[idx] *= np.float32(outlier_mult)
    return to_f16_bits(v)


def weight_rowscaled_f16_bits(N: int, K: int, seed: int, sigma: float = 0.02) -> np.ndarray:
    """fp16 weight bit patterns [N, K] ~ N(0, sigma^2) with row r scaled by
    2^((5 r mod 11) - 5) in float32 before the fp16 cast: neighbouring rows
    differ in magnitude by up to 2^10, so per-block constants differ widely
    from row to row and from one run of blocks to the next."""
    v = normal_f32((N, K), seed, sigma, 0.0)
    e = ((5 * np.arange(N)) % 11 - 5).astype(np.float32)
    v *= np.exp2(e)[:, None].astype(np.float32)
    return to_f16_bits(v)


def act_bits(M: int, K: int, seed: int, act_t: int) -> np.ndarray:
    """Activation bit patterns [M, K] ~ N(0, 1) in fp16 (F16) or bf16 (BF16)."""
    v = normal_f32((M, K), seed)
    return to_f16_bits(v) if act_t == F16 else to_bf16_bits(v)


# The five workloads: format, group, shapes, seeds and value distributions.
CONFIGS = {
    "c1_nf4_1k": dict(fmt=NF4, g=64, act=F16, mats=[(1024, 1024, 101)], x_seeds=[102],
                      M=[1], sigma=0.02, mu=0.0),
    "c2_sym_4k": dict(fmt=INT4_SYM, g=128, act=F16, mats=[(4096, 4096, 201)], x_seeds=[203],
                      M=[1], sigma=0.02, mu=0.0, outlier_seed=202),
    "c3_nf4_mlp": dict(fmt=NF4, g=64, act=BF16, mats=[(11008, 4096, 301), (4096, 11008, 302)],
                       x_seeds=[303, 304], M=[1, 4, 16], sigma=0.02, mu=0.0),
    "c4_asym_gemm": dict(fmt=INT4_ASYM, g=32, act=BF16, mats=[(14336, 4096, 401)], x_seeds=[402],
                         M=[2048], sigma=0.02, mu=0.001),
}

# The 7B-style decoder stack: per layer q, k, v, o (4096x4096), gate, up
# (11008x4096) and down (4096x11008); weight seed 5000 + 7*layer + index.
LLAMA7B_LAYER = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
                 ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)]
LLAMA7B_LAYERS = 32


def llama7b_seed(layer: int, idx: int) -> int:
    return 5000 + 7 * layer + idx
