"""Helpers of the GPU parity tests (no test functions here)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> device bfloat16 tensor, bit for bit."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f32(host_bf16_bits(t)).astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    """||a - b||_F / ||b||_F in float64; a must be exactly zero where ||b|| = 0."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    if nb == 0.0:
        return 0.0 if np.all(a == 0.0) else float("inf")
    return float(np.linalg.norm(a - b) / nb)


def segments_of(offsets: np.ndarray, rows: int) -> np.ndarray:
    """Expert id of each permuted row r < offsets[-1] (int32 [rows])."""
    eor = np.full(rows, -1, dtype=np.int32)
    for e in range(len(offsets) - 1):
        eor[offsets[e]:offsets[e + 1]] = e
    return eor


def sample_tokens(T: int, n: int, seed: int) -> np.ndarray:
    """n distinct tokens spread over [0, T) plus the first and the last."""
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(T, size=min(n, T), replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(pick), dtype=np.int64)
