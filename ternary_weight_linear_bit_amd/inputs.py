"""Seeded synthetic inputs and workload shapes.

This module only draws random numbers and describes shapes.  It holds none of
the quantisation or matmul arithmetic, so both the HIP path and the CPU oracle
can be fed from it without sharing any of the method's code.

Value distributions: master weights ~ N(0, 0.02^2) in fp32, activations
~ N(0, 1) (optionally rounded to bf16 by torch).  Seeds: weight matrix i of
layer l uses 1000 + 7*l + i, activations use 7 unless a caller says otherwise.

Layer shapes follow the models the pages name: BitNet b1.58 2B4T (hidden 2560,
kv 640, FFN 6912, 30 layers) and the Llama-3-8B-shaped 1.58-bit model (hidden
4096, kv 1024, FFN 14336), plus a ~100B-class stack (hidden 8192, FFN 28672,
96 layers) sized like the 100B model the pages run on one CPU.
"""

from __future__ import annotations

import numpy as np

WEIGHT_SIGMA = 0.02
ACT_SEED = 7


def weight_seed(layer: int, index: int) -> int:
    return 1000 + 7 * layer + index


def master_weights(n: int, k: int, seed: int, sigma: float = WEIGHT_SIGMA) -> np.ndarray:
    """fp32 [N, K] ~ N(0, sigma^2) from numpy's PCG64 with the given seed."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((n, k), dtype=np.float32) * np.float32(sigma)


def ternary_codes(n: int, k: int, seed: int) -> np.ndarray:
    """int8 [N, K] in {-1, 0, +1} with the mix of absmean-ternarised N(0, sigma)
    weights, P(0) = 0.31 and P(+1) = P(-1) = 0.345 (numpy PCG64, seeded): ready-made
    ternary weights for shapes too large to ternarise master weights on the host."""
    u = np.random.Generator(np.random.PCG64(seed)).random((n, k), dtype=np.float32)
    return (u > np.float32(0.655)).astype(np.int8) - (u < np.float32(0.345)).astype(np.int8)


def activations(m: int, k: int, seed: int = ACT_SEED) -> np.ndarray:
    """fp32 [M, K] ~ N(0, 1) from numpy's PCG64 with the given seed."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((m, k), dtype=np.float32)


def norm_weight(k: int, seed: int) -> np.ndarray:
    """Seeded RMS norm weights [K] fp32: 1 + 0.1 * N(0, 1) (synthetic stand-ins for
    trained ones)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (1.0 + 0.1 * rng.standard_normal(k)).astype(np.float32)


def to_bf16(x_f32: np.ndarray):
    """Round an fp32 array to a torch bf16 CPU tensor (torch's own conversion)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x_f32)).to(torch.bfloat16)


# (name, K, N) of each ternary matrix in one layer; N = output features.
LAYER_2B = (("q", 2560, 2560), ("k", 2560, 640), ("v", 2560, 640), ("o", 2560, 2560),
            ("gate", 2560, 6912), ("up", 2560, 6912), ("down", 6912, 2560))
LAYER_8B = (("q", 4096, 4096), ("k", 4096, 1024), ("v", 4096, 1024), ("o", 4096, 4096),
            ("gate", 4096, 14336), ("up", 4096, 14336), ("down", 14336, 4096))
LAYER_100B = (("q", 8192, 8192), ("k", 8192, 8192), ("v", 8192, 8192), ("o", 8192, 8192),
              ("gate", 8192, 28672), ("up", 8192, 28672), ("down", 28672, 8192))

WORKLOADS = {
    "single-256x256-m4": dict(layer=(("w", 256, 256),), layers=1, m=(4,), act="f32"),
    "bitnet2b-decode-m1-30L": dict(layer=LAYER_2B, layers=30, m=(1,), act="bf16"),
    "bitnet2b-prefill": dict(layer=LAYER_2B, layers=1, m=(512, 4096), act="bf16"),
    "llama8b-ternary": dict(layer=LAYER_8B, layers=32, m=(1, 16, 2048), act="bf16"),
    "ternary100b-decode-m1-96L": dict(layer=LAYER_100B, layers=96, m=(1,), act="f32"),
    "ternary100b-decode-m1-96L-bf16": dict(layer=LAYER_100B, layers=96, m=(1,), act="bf16"),
}


def packed_bytes(layer_shapes, fmt: str = "2bit") -> int:
    """Packed weight bytes of one layer: N*K/4 (2 bits per weight) or
    N*16*ceil(K/80) (five weights per byte)."""
    if fmt == "t1":
        return sum(n * 16 * ((k + 79) // 80) for _, k, n in layer_shapes)
    return sum(n * k // 4 for _, k, n in layer_shapes)
