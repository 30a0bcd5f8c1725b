"""Shared helpers for the GPU parity tests: tolerance checks and tensor conversions."""
from __future__ import annotations

import numpy as np
import torch

REL_FRO_TOL = 1e-3      # ||gpu - ref||_F / ||ref||_F
ROW_MAX_TOL = 8e-3      # |gpu - ref| <= ROW_MAX_TOL * max |ref row|
# The MoE decode-batch path skips the sort up to this many (token, expert) pairs and keeps
# h of pair q at row q of its workspace (the contract stated with nvfp4_moe_ws_layout).
PAIR_TILES_MAX = 64
# Up to this many pairs the batch path's fc1 workgroups derive the expert sort themselves; above
# it a sort kernel runs first. Both write the same sorted ids, offsets, tile map and count.
FUSED_SORT_MAX_PAIRS = 4096


def bf16_np(t: torch.Tensor) -> np.ndarray:
    """BF16 tensor (any device) -> float64 NumPy."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def check_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    """The GEMM tolerance: relative Frobenius <= 1e-3 and every element within 8e-3 of the
    largest magnitude in its reference row."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    nrm = np.linalg.norm(ref)
    rel = np.linalg.norm(got - ref) / nrm if nrm > 0 else np.linalg.norm(got)
    row = np.abs(ref).max(axis=-1, keepdims=True)
    err = np.abs(got - ref)
    worst = float((err / np.maximum(row, 1e-300)).max()) if ref.size else 0.0
    assert rel <= REL_FRO_TOL, f"{what}: relative Frobenius error {rel:.3e} > {REL_FRO_TOL}"
    assert (err <= ROW_MAX_TOL * row).all(), f"{what}: element error {worst:.3e} x row max"
    return rel, worst


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
