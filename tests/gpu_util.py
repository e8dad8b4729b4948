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


def host_f64(t: torch.Tensor, rows=None) -> np.ndarray:
    """The tensor in float64 on the host; with `rows` (an index or slice of the
    first dimension), only those rows, selected before widening so that
    unwritten rows (possibly signaling-NaN patterns) are never converted."""
    if t.dtype == torch.bfloat16:
        bits = host_bf16_bits(t)
        if rows is not None:
            bits = bits[rows]
        return synth.bf16_bits_to_f32(bits).astype(np.float64)
    a = t.detach().cpu().numpy()
    if rows is not None:
        a = a[rows]
    return a.astype(np.float64)


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


def covering_tokens(local_ids: np.ndarray, n: int, seed: int) -> np.ndarray:
    """Tokens to check at full size: for every local expert that any route
    reaches, at least one chosen token routes to it (greedy over the tokens in
    a seeded random order), then random tokens up to n in all, plus the first
    and the last token.  local_ids: int [T, k], the local expert of each
    route (-1: not local)."""
    T = local_ids.shape[0]
    rng = np.random.default_rng(seed)
    order = rng.permutation(T)
    pick = {0, T - 1}
    need = set(int(e) for e in np.unique(local_ids) if e >= 0)
    for t in pick:
        need -= set(int(e) for e in local_ids[t])
    for t in order:
        if not need:
            break
        s = set(int(e) for e in local_ids[t]) & need
        if s:
            pick.add(int(t))
            need -= s
    assert not need
    for t in order:
        if len(pick) >= n:
            break
        pick.add(int(t))
    return np.array(sorted(pick), dtype=np.int64)


def per_row_rel(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """||got_r - ref_r|| / ||ref_r|| for every row r (float64); a row whose
    reference is all zero must be exactly zero (0 if so, inf if not)."""
    got = np.asarray(got, dtype=np.float64).reshape(got.shape[0], -1)
    ref = np.asarray(ref, dtype=np.float64).reshape(ref.shape[0], -1)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    out = np.empty_like(num)
    z = den == 0.0
    out[~z] = num[~z] / den[~z]
    out[z] = np.where(np.all(got[z] == 0.0, axis=1), 0.0, np.inf)
    return out


def expert_sample_rows(offsets: np.ndarray, per_expert: int, seed: int) -> np.ndarray:
    """Permuted rows to check at full size: for every local expert with rows,
    its first and last row and up to per_expert - 2 more at random (so every
    expert, and for long segments several of its m-tiles, is covered)."""
    rng = np.random.default_rng(seed)
    rows = []
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            continue
        sel = {lo, hi - 1}
        if hi - lo > 2 and per_expert > 2:
            extra = rng.choice(np.arange(lo + 1, hi - 1), size=min(per_expert - 2, hi - lo - 2),
                               replace=False)
            sel.update(int(r) for r in extra)
        rows.extend(sorted(sel))
    return np.array(rows, dtype=np.int64)
