"""Seeded synthetic inputs for the Sherry layer (shared by tests, bench, smoke).

This module holds none of the method's arithmetic: it draws latent weights and
activations, rounds activations to bf16 (input preparation), and names the
workload shapes.  Both the CPU oracle and the HIP path receive the exact same
bytes from here.

Shapes: LLaMA-3.2-1B and -3B decoder-layer linears in ``nn.Linear`` ``[N, K]``
order (N = out_features, K = in_features).  The pages train and evaluate on
these two models with group size 128 (Sherry digest, Arenas paragraph).  No
trained weights or datasets are used: weights are N(0, 0.02) and activations
N(0, 1), as stated for each workload below.
"""

from __future__ import annotations

import numpy as np

# (name, N, K)
LLAMA_1B = (
    ("q", 2048, 2048), ("k", 512, 2048), ("v", 512, 2048), ("o", 2048, 2048),
    ("gate", 8192, 2048), ("up", 8192, 2048), ("down", 2048, 8192),
)
LLAMA_3B = (
    ("q", 3072, 3072), ("k", 1024, 3072), ("v", 1024, 3072), ("o", 3072, 3072),
    ("gate", 8192, 3072), ("up", 8192, 3072), ("down", 3072, 8192),
)
LLAMA_3B_LAYERS = 28
GROUP = 128

# Seeds.  Single layer: W 0, x 1.  1B layer: W 100+i, x 200.  3B stack:
# W 1000 + 7*layer + i, x 2000 + B.  Prefill: X 300 + M.  Quantize: 5000.
SEED_SMALL_W, SEED_SMALL_X = 0, 1


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 bit patterns, nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return (r & np.uint64(0xFFFF)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def latent_weight(n: int, k: int, seed: int, std: float = 0.02) -> np.ndarray:
    """fp32 latent weight ~ N(0, std^2), ``[N, K]``."""
    return rng(seed).standard_normal((n, k), dtype=np.float32) * np.float32(std)


def latent_weight_outliers_bf16(n: int, k: int, seed: int, std: float = 0.02,
                                frac: float = 0.01, factor: float = 10.0):
    """bf16 latent weight with outliers: N(0, std^2) in fp32, exactly
    ``round(frac*N*K)`` positions (drawn without replacement) scaled by
    ``factor`` in fp32, then the whole matrix rounded to bf16 (nearest-even).

    Returns ``(bits uint16 [N,K], values fp32 [N,K])``; the fp32 values are the
    exact widening of the bf16 bits.
    """
    g = rng(seed)
    w = g.standard_normal((n, k), dtype=np.float32) * np.float32(std)
    count = int(round(frac * n * k))
    idx = g.choice(n * k, size=count, replace=False)
    flat = w.reshape(-1)
    flat[idx] = flat[idx] * np.float32(factor)
    bits = f32_to_bf16_bits(w)
    return bits, bf16_bits_to_f32(bits)


def activations_bf16(rows: int, k: int, seed: int):
    """bf16 activations ~ N(0, 1): ``(bits uint16 [rows,K], fp32 values)``."""
    x = rng(seed).standard_normal((rows, k), dtype=np.float32)
    bits = f32_to_bf16_bits(x)
    return bits, bf16_bits_to_f32(bits)


def layer_1b_weight_seed(i: int) -> int:
    return 100 + i


def layer_3b_weight_seed(layer: int, i: int) -> int:
    return 1000 + 7 * layer + i


def latent_weight_device(n: int, k: int, seed: int, device, std: float = 0.02):
    """fp32 latent weight ~ N(0, std^2) drawn on the GPU with torch's seeded
    Philox generator (for the 28-layer 3B stack, where host generation would
    dominate the run).  Checks copy the same bytes back to the host."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn((n, k), generator=g, device=device, dtype=torch.float32) * std
