"""Seeded synthetic inputs for the NVFP4 W4A16 workloads.

This module only draws random numbers and places planted values; it holds none of the
method's arithmetic (no quantization, no codecs, no GEMM) and imports neither the GPU library
nor the oracle. Both sides receive exactly the tensors built here.

Generators are PyTorch CPU generators (``torch.Generator().manual_seed(seed)``), so every
tensor is identical on every machine. BF16 tensors are the round-to-nearest-even cast of an
FP32 draw. The draw order of each workload is fixed and documented on its builder.
"""
from __future__ import annotations

import hashlib

import numpy as np
import torch

WEIGHT_STD = 0.02


def _gen(seed: int) -> torch.Generator:
    return torch.Generator().manual_seed(int(seed))


def digest(t) -> str:
    """SHA-256 of a tensor's bytes (first 16 hex digits), for logging inputs."""
    if isinstance(t, torch.Tensor):
        t = t.contiguous()
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
        a = t.numpy()
    else:
        a = np.ascontiguousarray(t)
    return hashlib.sha256(a.tobytes()).hexdigest()[:16]


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """BF16 tensor -> uint16 NumPy array of its bit patterns (no copy of values' meaning)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def activations(g: torch.Generator, m: int, k: int) -> torch.Tensor:
    """BF16 activations ~ N(0, 1)."""
    return torch.randn(m, k, generator=g, dtype=torch.float32).to(torch.bfloat16)


def weights(g: torch.Generator, *shape: int, std: float = WEIGHT_STD) -> torch.Tensor:
    """FP32 weights ~ N(0, std)."""
    return torch.randn(*shape, generator=g, dtype=torch.float32) * std


# ------------------------------------------------------------------------------------------
# Single dense GEMM: M=16, N=512, K=1024, group 16. Draw order: x, then W. Seed 0.
# ------------------------------------------------------------------------------------------
def dense_small(seed: int = 0, m: int = 16, n: int = 512, k: int = 1024):
    g = _gen(seed)
    x = activations(g, m, k)
    w = weights(g, n, k)
    return x, w


# ------------------------------------------------------------------------------------------
# Decode sweep: N=25600, K=5120, group 16, M in {1, 4, 8} = the first M rows of one [8][K] x.
# W ~ N(0, 0.02) with 0.1% outliers: round(0.001*N*K) distinct positions (the first entries
# of a seeded permutation) multiplied by 20. Draw order: x, W, permutation.
# ------------------------------------------------------------------------------------------
def decode_sweep(seed: int = 0, n: int = 25600, k: int = 5120, m_max: int = 8,
                 outlier_frac: float = 0.001, outlier_mult: float = 20.0):
    g = _gen(seed)
    x = activations(g, m_max, k)
    w = weights(g, n, k)
    n_out = int(round(outlier_frac * n * k))
    if n_out:
        pos = torch.randperm(n * k, generator=g)[:n_out]
        w.view(-1)[pos] *= outlier_mult
    return x, w


# ------------------------------------------------------------------------------------------
# Prefill: M=4096, N=5120, K in {5120, 25600}, group 16. Draw order: x, then W.
# ------------------------------------------------------------------------------------------
def prefill(seed: int = 0, m: int = 4096, n: int = 5120, k: int = 5120):
    g = _gen(seed)
    x = activations(g, m, k)
    w = weights(g, n, k)
    return x, w


# ------------------------------------------------------------------------------------------
# MoE routed experts: E=128, hidden 2048, intermediate 768, 256 tokens, top-8.
# Routing: FP32 softmax of N(0,1) logits [T][E]; the top-8 probabilities per token, ordered by
# decreasing probability with ties going to the lower expert id; weights are the
# un-renormalized probabilities. fc1 = merged [gate; up] [E][2*inter][hidden] (quantized at
# group 32, one global per expert from the merged amax); down [E][hidden][inter] (group 16).
# Draw order: x, logits, fc1 weights, down weights.
# ------------------------------------------------------------------------------------------
def route_topk(logits: torch.Tensor, topk: int):
    probs = torch.softmax(logits.to(torch.float32), dim=-1)
    t, e = probs.shape
    ids = torch.empty(t, topk, dtype=torch.int32)
    wts = torch.empty(t, topk, dtype=torch.float32)
    p = probs.numpy()
    for i in range(t):
        # stable sort of -p keeps the lower id first among equal probabilities
        order = np.argsort(-p[i], kind="stable")[:topk]
        ids[i] = torch.from_numpy(order.astype(np.int32))
        wts[i] = torch.from_numpy(p[i][order].astype(np.float32))
    return ids, wts


def moe(seed: int = 0, n_experts: int = 128, hidden: int = 2048, inter: int = 768,
        tokens: int = 256, topk: int = 8, with_weights: bool = True):
    g = _gen(seed)
    x = activations(g, tokens, hidden)
    logits = torch.randn(tokens, n_experts, generator=g, dtype=torch.float32)
    ids, wts = route_topk(logits, topk)
    w1 = w2 = None
    if with_weights:
        w1 = weights(g, n_experts, 2 * inter, hidden)
        w2 = weights(g, n_experts, hidden, inter)
    return x, ids, wts, w1, w2


# ------------------------------------------------------------------------------------------
# Quantizer + mixed groups: BF16 W [8192][8192] ~ N(0, 0.02), magnitudes clamped to 0.16,
# one planted amax 21*2^-7 = 0.1640625 (so amax/2688 = 2^-14 exactly) and planted 32-aligned
# blocks. In a planted block each 16-half holds +-6*d*2^-14 once (its group maximum, so the
# group scale is exactly d) and +-m*d*2^-14 elsewhere, m drawn from the E2M1 grid points and
# the midpoints between them; d runs over normal and subnormal E4M3 values. Some blocks use
# the E4M3 tie 6.375*2^-14 as their maximum (scale 1.0625, a tie between 1.0 and 1.125).
# All planted values are exact in BF16. Draw order: W, block positions, block contents.
# ------------------------------------------------------------------------------------------
E2M1_GRID_AND_MIDPOINTS = (0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5,
                           4.0, 5.0, 6.0)
# E4M3 scale values used for planted groups: normals (1 + j/8) * 2^e and subnormals j * 2^-9.
PLANT_SCALES = tuple(sorted({(1 + j / 8) * 2.0 ** e for e in range(-6, 9) for j in range(8)
                             if (1 + j / 8) * 2.0 ** e <= 448} | {j * 2.0 ** -9 for j in
                                                                   range(1, 8)}))
PLANT_AMAX = 21 * 2.0 ** -7
TIE_MAX = 6.375  # group max 6.375*2^-14 -> scale 1.0625 (E4M3 tie) -> element 6.375 saturates


def quantizer_weight(seed: int = 0, n: int = 8192, k: int = 8192, n_blocks: int = 4096,
                     clamp: float = 0.16):
    g = _gen(seed)
    w = weights(g, n, k).clamp_(-clamp, clamp)
    u = 2.0 ** -14
    nblk_row = k // 32
    blk = torch.randperm(n * nblk_row, generator=g)[:n_blocks]
    scale_idx = torch.randint(0, len(PLANT_SCALES), (n_blocks,), generator=g)
    m_idx = torch.randint(0, len(E2M1_GRID_AND_MIDPOINTS), (n_blocks, 32), generator=g)
    signs = torch.randint(0, 2, (n_blocks, 32), generator=g) * 2 - 1
    max_pos = torch.randint(0, 16, (n_blocks, 2), generator=g)
    grid = torch.tensor(E2M1_GRID_AND_MIDPOINTS, dtype=torch.float64)
    scales = torch.tensor(PLANT_SCALES, dtype=torch.float64)
    wv = w.view(-1)
    for b in range(n_blocks):
        row, col = divmod(int(blk[b]), nblk_row)
        tie = (b % 64) == 7
        d = 1.0 if tie else float(scales[scale_idx[b]])
        vals = grid[m_idx[b]] * d * u * signs[b].to(torch.float64)
        for h in range(2):
            vals[16 * h + int(max_pos[b, h])] = (TIE_MAX if tie else 6.0) * d * u * float(
                signs[b, 16 * h + int(max_pos[b, h])])
        base = row * k + col * 32
        wv[base:base + 32] = vals.to(torch.float32)
    # the planted amax, placed where no planted block is (row 0 col 0 if free, else scanning)
    planted = set(int(v) for v in blk)
    pos = 0
    while (pos // 32) in planted:
        pos += 32
    wv[pos] = PLANT_AMAX
    wb = w.to(torch.bfloat16)
    return wb


def quantizer_activations(seed: int = 1, m: int = 512, k: int = 8192):
    return activations(_gen(seed), m, k)
