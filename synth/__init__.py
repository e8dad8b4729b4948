"""Seeded synthetic inputs for the fused MoE layer (shared by tests and bench).

Every value is a pure function of (seed, tensor_id, element index), drawn by
the counter-based generator in ``synth.c`` (SplitMix64 + Box-Muller).  This
module holds no MoE arithmetic: it draws numbers, rounds them to the storage
dtype and packs MXFP4 weights.  bf16 tensors are returned as ``numpy.uint16``
bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

# Tensor ids of the input streams.
TID_X, TID_LOGITS, TID_W1, TID_W2, TID_WS1, TID_WS2 = 0, 1, 2, 3, 4, 5


def build(force: bool = True) -> str:
    """Compile ``synth.c`` into ``libsynth.so`` next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.synth_splitmix64.restype = u64
        lib.synth_splitmix64.argtypes = [u64]
        lib.synth_raw_u64.restype = u64
        lib.synth_raw_u64.argtypes = [u64, u64, u64]
        lib.synth_normal_at.restype = dbl
        lib.synth_normal_at.argtypes = [u64, u64, u64]
        lib.synth_normal_f32.restype = None
        lib.synth_normal_f32.argtypes = [u64, u64, i64, dbl, dbl, vp]
        lib.synth_normal_bf16.restype = None
        lib.synth_normal_bf16.argtypes = [u64, u64, i64, dbl, dbl, vp]
        lib.synth_biased_logits.restype = None
        lib.synth_biased_logits.argtypes = [u64, u64, i64, i64, vp, vp]
        lib.synth_mxfp4_quantize.restype = None
        lib.synth_mxfp4_quantize.argtypes = [vp, i64, i64, vp, vp]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def splitmix64(x: int) -> int:
    """SplitMix64 output for state x: mix(x + golden gamma)."""
    return int(_load().synth_splitmix64(x))


def raw_u64(seed: int, tensor_id: int, i: int) -> int:
    return int(_load().synth_raw_u64(seed, tensor_id, i))


def normal_at(seed: int, tensor_id: int, i: int) -> float:
    return float(_load().synth_normal_at(seed, tensor_id, i))


def normal_f32(seed: int, tensor_id: int, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().synth_normal_f32(seed, tensor_id, out.size, mean, std, _ptr(out))
    return out


def normal_bf16(seed: int, tensor_id: int, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint16)
    _load().synth_normal_bf16(seed, tensor_id, out.size, mean, std, _ptr(out))
    return out


def biased_logits(seed: int, tensor_id: int, T: int, bias: np.ndarray) -> np.ndarray:
    bias = np.ascontiguousarray(bias, dtype=np.float64)
    E = bias.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    _load().synth_biased_logits(seed, tensor_id, T, E, _ptr(bias), _ptr(out))
    return out


def zipf_log_bias(E: int, s: float) -> np.ndarray:
    """ln p_e with p_e proportional to (e+1)^-s (expert 0 most popular)."""
    p = (np.arange(1, E + 1, dtype=np.float64)) ** (-s)
    p /= p.sum()
    return np.log(p)


def mxfp4_quantize(w_bf16: np.ndarray):
    """bf16 bits [..., K] -> (packed uint8 [..., K/2], E8M0 scales uint8 [..., K/32])."""
    K = w_bf16.shape[-1]
    if K % 32:
        raise ValueError("MXFP4 needs K to be a multiple of 32")
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    rows = w.size // K
    packed = np.empty(w.shape[:-1] + (K // 2,), dtype=np.uint8)
    scales = np.empty(w.shape[:-1] + (K // 32,), dtype=np.uint8)
    _load().synth_mxfp4_quantize(_ptr(w), rows, K, _ptr(packed), _ptr(scales))
    return packed, scales


def fp8_quantize_rows(w_bf16: np.ndarray):
    """Test weights in FP8 E4M3 with one float32 scale per row (per output
    channel): bf16 bits [..., K] -> (codes uint8 [..., K], scales float32 [...]).
    scale = amax / 448 of the row (1 for an all-zero row); the codes are torch's
    round-to-nearest-even cast of w / scale, clamped to +-448 first."""
    import torch
    w = bf16_bits_to_f32(np.ascontiguousarray(w_bf16, dtype=np.uint16))
    amax = np.abs(w).max(axis=-1)
    scales = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    v = np.clip(w / scales[..., None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scales


def fp8_quantize_blocks(w_bf16: np.ndarray, block: int = 128):
    """Test weights in block-scaled FP8 E4M3: bf16 bits [..., N, K] -> (codes
    uint8 [..., N, K], scales float32 [..., N/block, K/block]), one scale per
    block x block tile: amax / 448 of the tile (1 for an all-zero tile); the
    codes are torch's round-to-nearest-even cast of w / scale, clamped first."""
    import torch
    w = bf16_bits_to_f32(np.ascontiguousarray(w_bf16, dtype=np.uint16))
    *lead, N, K = w.shape
    if N % block or K % block:
        raise ValueError("N and K must be multiples of the block")
    t = w.reshape(*lead, N // block, block, K // block, block)
    amax = np.abs(t).max(axis=(-3, -1))
    scales = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    v = np.clip(t / scales[..., :, None, :, None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(np.ascontiguousarray(v)).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.numpy().reshape(w.shape), scales


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (bit shift, no arithmetic)."""
    return (a.astype(np.uint32) << 16).view(np.float32)
