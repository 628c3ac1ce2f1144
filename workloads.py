"""Seeded synthetic inputs for the BitLinear forward, shared by tests and bench.

This module holds only input generation (random draws and one fp32 -> bf16
cast of the raw draws); it contains none of the method's arithmetic, so that
the oracle and the HIP path can both be fed byte-identical inputs from it.

Recipe (all on the host, torch CPU generator, one generator per draw):
  * latent weights W[N][K]: fp32 N(0, 0.02^2)  (0.02 read as the std);
  * activations X[M][K]: fp32 N(0, 1), optionally with 1% outliers (each
    element independently, Bernoulli(0.01), multiplied by 20 in fp32), then one
    round-to-nearest-even cast to bf16;
  * seeds: every workload uses seed 0 for its first tensor; the i-th tensor a
    workload draws uses seed ``base + i`` so tensors are independent.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

W_STD = 0.02


def gen_weights(N: int, K: int, seed: int, std: float = W_STD) -> np.ndarray:
    """Latent fp32 weights [N][K] ~ N(0, std^2)."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    w = torch.randn((N, K), generator=g, dtype=torch.float32) * std
    return w.numpy()


def gen_acts_bf16(M: int, K: int, seed: int, outliers: bool = False) -> np.ndarray:
    """bf16 activations [M][K] ~ N(0, 1) as uint16 bit patterns.

    With ``outliers``, 1% of the elements (Bernoulli(0.01), drawn after the
    Gaussian) are multiplied by 20 before the bf16 cast.
    """
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    x = torch.randn((M, K), generator=g, dtype=torch.float32)
    if outliers:
        mask = torch.rand((M, K), generator=g) < 0.01
        x = torch.where(mask, x * 20.0, x)
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 values."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------- configs
@dataclass(frozen=True)
class Linear:
    """One BitLinear shape: M tokens, K inputs, N outputs."""
    M: int
    K: int
    N: int
    outliers: bool = False


@dataclass(frozen=True)
class Workload:
    name: str
    linears: tuple = field(default_factory=tuple)


# Single BitLinear, 4 tokens, 512 -> 512, seed 0.
SINGLE_4x512 = Workload("single_4x512x512", (Linear(4, 512, 512),))

# Decode GEMV at batch 1 on the 2B-class shapes, activations with 1% x20 outliers.
DECODE_2B = Workload("decode_gemv_2b_m1", (Linear(1, 2560, 6912, True), Linear(1, 6912, 2560, True)))

# 2B-class decoder layer: d=2560, FFN 6912, 20 query heads / 5 kv heads of dim 128.
D_MODEL, D_FFN, N_LAYERS, HEAD_DIM, N_Q_HEADS, N_KV_HEADS = 2560, 6912, 30, 128, 20, 5
LAYER_SHAPES = (
    ("q", D_MODEL, N_Q_HEADS * HEAD_DIM),
    ("k", D_MODEL, N_KV_HEADS * HEAD_DIM),
    ("v", D_MODEL, N_KV_HEADS * HEAD_DIM),
    ("o", N_Q_HEADS * HEAD_DIM, D_MODEL),
    ("gate", D_MODEL, D_FFN),
    ("up", D_MODEL, D_FFN),
    ("down", D_FFN, D_MODEL),
)

# One decode step over every BitLinear of the 30-layer stack, batch 1 and 8.
DECODE_STEP_BATCHES = (1, 8)


def decoder_weight_seed(layer: int, j: int) -> int:
    """Seed of the j-th matrix (LAYER_SHAPES order) of decoder layer ``layer``."""
    return 100 + 7 * layer + j


DECODER_X0_SEED = 1  # seed of the bf16 input tokens of the decode step


# Prefill GEMM: 2048 tokens on the 2B-class FFN shapes.
PREFILL_2B = Workload("prefill_gemm_2b_m2048", (Linear(2048, 2560, 6912), Linear(2048, 6912, 2560)))

# 100B-class layer shapes.
SHAPES_100B = ((8192, 28672), (28672, 8192))


# Decode GEMV at batch 1 on the 100B-class shapes (the largest configuration
# that fits one GPU), activations bf16 N(0, 1).
DECODE_100B = Workload("decode_gemv_100b_m1", tuple(Linear(1, K, N) for K, N in SHAPES_100B))


def workload_100b(M: int) -> Workload:
    return Workload("shapes_100b_m%d" % M, tuple(Linear(M, K, N) for K, N in SHAPES_100B))
