"""CPU oracle for the fused MoE layer (ctypes wrapper over ``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke()``
and by the benchmark's ``cpu_baseline`` leg, never by the product package.  It
shares no code with the HIP library.  All floating-point results are float64.

Parity pins (what fixes each function independently of itself) live in
``tests/test_oracle_*.py``.  No function here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

SOFTMAX, SIGMOID = 0, 1
W_BF16, W_MXFP4, W_FP8, W_FP8_BLOCK = 0, 1, 2, 3
BLOCK = 128  # rows and columns of a weight block, elements of an activation group
ACTIVATIONS = {"silu": 0, "gelu": 1}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP) into ``liboracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _W(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("data", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        vp, i64, i32, dbl, u8 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                 ctypes.c_double, ctypes.c_uint8)
        Wp = ctypes.POINTER(_W)
        L.oracle_e8m0_scale.restype = dbl
        L.oracle_e8m0_scale.argtypes = [u8]
        L.oracle_mxfp4_value.restype = dbl
        L.oracle_mxfp4_value.argtypes = [vp, vp, i64, i64, i64]
        L.oracle_route.restype = None
        L.oracle_route.argtypes = [vp, i64, i32, i32, i32, i32, dbl, vp, vp]
        L.oracle_permute.restype = ctypes.c_int
        L.oracle_permute.argtypes = [vp, vp, i64, i32, i32, i32, vp, vp, vp]
        L.oracle_permute_batched.restype = ctypes.c_int
        L.oracle_permute_batched.argtypes = [vp, vp, i64, i32, i32, i32, i32, vp, vp]
        L.oracle_hidden_rows.restype = None
        L.oracle_hidden_rows.argtypes = [vp, i64, i64, i64, Wp, vp, i32, dbl, vp]
        L.oracle_e4m3_decode.restype = dbl
        L.oracle_e4m3_decode.argtypes = [u8]
        L.oracle_e4m3_encode.restype = u8
        L.oracle_e4m3_encode.argtypes = [dbl]
        L.oracle_quantize_fp8_rows.restype = None
        L.oracle_quantize_fp8_rows.argtypes = [vp, i64, i64, vp, vp, vp]
        L.oracle_quantize_fp8x2_rows.restype = None
        L.oracle_quantize_fp8x2_rows.argtypes = [vp, i64, i64, vp, vp, vp]
        L.oracle_hidden_rows_fp8.restype = None
        L.oracle_hidden_rows_fp8.argtypes = [vp, vp, i64, i64, i64, i64, Wp, vp, i32, dbl, vp]
        L.oracle_out_rows_fp8.restype = None
        L.oracle_out_rows_fp8.argtypes = [vp, vp, i64, i64, i64, i64, Wp, vp, vp]
        L.oracle_quantize_fp8_groups.restype = None
        L.oracle_quantize_fp8_groups.argtypes = [vp, i64, i64, i64, vp, vp]
        L.oracle_hidden_rows_fp8x2.restype = None
        L.oracle_hidden_rows_fp8x2.argtypes = [vp, vp, vp, i64, i64, i64, Wp, vp, i32, dbl, vp]
        L.oracle_out_rows_fp8x2.restype = None
        L.oracle_out_rows_fp8x2.argtypes = [vp, vp, vp, i64, i64, i64, Wp, vp, vp]
        L.oracle_out_rows.restype = None
        L.oracle_out_rows.argtypes = [vp, i64, i64, i64, Wp, vp, vp]
        L.oracle_finalize.restype = None
        L.oracle_finalize.argtypes = [vp, vp, vp, i64, i32, i64, dbl, vp, vp]
        L.oracle_finalize_add_rmsnorm.restype = None
        L.oracle_finalize_add_rmsnorm.argtypes = [vp, vp, vp, i64, i32, i64, dbl, vp, vp, vp, dbl,
                                                  vp, vp]
        L.oracle_moe_tokens.restype = None
        L.oracle_moe_tokens.argtypes = [vp, i64, i64, vp, i32, i32, i32, i32, dbl, vp, Wp, Wp,
                                        i64, vp, vp, dbl, i32, dbl, i32, i32, vp, vp, vp, i64, vp,
                                        vp, vp, vp]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_num_threads.argtypes = []
        _lib = L
    return _lib


def _c(a: Optional[np.ndarray], dtype) -> Optional[np.ndarray]:
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


class Weights:
    """Expert weights in bf16 bits ([rows, K] uint16), MXFP4 (packed uint8
    [rows, K/2] + E8M0 uint8 [rows, K/32]), FP8 E4M3 (uint8 [rows, K] + one
    float32 scale per row) or, with block=True, block-scaled FP8 E4M3 (uint8
    [rows, K] + float32 [rows/128, K/128], one scale per 128 x 128 block).
    Keeps the arrays alive."""

    def __init__(self, data: np.ndarray, scales: Optional[np.ndarray] = None,
                 block: bool = False):
        if scales is None:
            self.data = _c(data, np.uint16)
            self.scales = None
            self.fmt = W_BF16
        elif block:
            self.data = _c(data, np.uint8)
            self.scales = _c(scales, np.float32)
            K = self.data.shape[-1]
            rows = self.data.size // K
            if rows % BLOCK or K % BLOCK or self.scales.size != (rows // BLOCK) * (K // BLOCK):
                raise ValueError("block FP8 weights need [rows/128, K/128] scales")
            self.fmt = W_FP8_BLOCK
        elif scales.dtype == np.float32:
            self.data = _c(data, np.uint8)
            self.scales = _c(scales, np.float32)
            self.fmt = W_FP8
        else:
            self.data = _c(data, np.uint8)
            self.scales = _c(scales, np.uint8)
            self.fmt = W_MXFP4
        self._s = _W(self.fmt, _p(self.data), _p(self.scales))

    @property
    def ref(self):
        return ctypes.byref(self._s)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def e8m0_scale(s: int) -> float:
    return float(_load().oracle_e8m0_scale(s))


def mxfp4_value(packed: np.ndarray, scales: np.ndarray, row: int, K: int, kk: int) -> float:
    packed, scales = _c(packed, np.uint8), _c(scales, np.uint8)
    return float(_load().oracle_mxfp4_value(_p(packed), _p(scales), row, K, kk))


def mxfp4_dequant(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Element-by-element decode of [rows, K/2] + [rows, K/32] -> float64 [rows, K]
    (small inputs only: one C call per element)."""
    packed, scales = _c(packed, np.uint8), _c(scales, np.uint8)
    rows, K = packed.shape[0], packed.shape[1] * 2
    out = np.empty((rows, K), dtype=np.float64)
    f = _load().oracle_mxfp4_value
    for r in range(rows):
        for kk in range(K):
            out[r, kk] = f(_p(packed), _p(scales), r, K, kk)
    return out


def route(logits: np.ndarray, k: int, score: int, renormalize: bool, rsf: float):
    """-> (ids int32 [T, k], weights float64 [T, k])."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    _load().oracle_route(_p(logits), T, E, k, score, int(bool(renormalize)), rsf, _p(ids), _p(w))
    return ids, w


def permute(ids: np.ndarray, E: int, E_l: int, expert_map: Optional[np.ndarray] = None):
    """-> (map int32 [T, k], offsets int32 [E_l+1], counts int32 [E_l]).
    Raises ValueError on ids outside [0, E) or map entries outside [-1, E_l)."""
    ids = _c(ids, np.int32)
    expert_map = _c(expert_map, np.int32)
    T, k = ids.shape
    m = np.empty((T, k), dtype=np.int32)
    offsets = np.empty(E_l + 1, dtype=np.int32)
    counts = np.empty(max(E_l, 1), dtype=np.int32)
    rc = _load().oracle_permute(_p(ids), _p(expert_map), T, k, E, E_l, _p(m), _p(offsets),
                                _p(counts))
    if rc != 0:
        raise ValueError("expert id out of range")
    return m, offsets, counts[:E_l]


def permute_batched(ids: np.ndarray, E: int, E_l: int, max_tokens: int,
                    expert_map: Optional[np.ndarray] = None):
    """Batched experts format -> (map int32 [T, k] into rows [E_l * max_tokens],
    counts int32 [E_l]).  Routes past an expert's capacity get -1."""
    ids = _c(ids, np.int32)
    expert_map = _c(expert_map, np.int32)
    T, k = ids.shape
    m = np.empty((T, k), dtype=np.int32)
    counts = np.empty(max(E_l, 1), dtype=np.int32)
    rc = _load().oracle_permute_batched(_p(ids), _p(expert_map), T, k, E, E_l, max_tokens, _p(m),
                                        _p(counts))
    if rc != 0:
        raise ValueError("expert id out of range")
    return m, counts[:E_l]


def e4m3_decode(code: int) -> float:
    return float(_load().oracle_e4m3_decode(code))


def e4m3_encode(v: float) -> int:
    return int(_load().oracle_e4m3_encode(float(v)))


def quantize_fp8_rows(x_bf16: np.ndarray, static_scale: Optional[float] = None):
    """Per-row FP8 E4M3 quantization of bf16 rows -> (codes uint8 [rows, H],
    scales float32 [rows]); static_scale: one given scale for every row."""
    x = _c(x_bf16, np.uint16)
    rows, H = x.shape
    q = np.empty((rows, H), dtype=np.uint8)
    sc = np.empty(rows, dtype=np.float32)
    st = None if static_scale is None else np.array([static_scale], dtype=np.float32)
    _load().oracle_quantize_fp8_rows(_p(x), rows, H, _p(st), _p(q), _p(sc))
    return q, sc


def quantize_fp8x2_rows(x_bf16: np.ndarray):
    """Two-term FP8 quantization of bf16 rows -> (q1 uint8 [rows, H], q2 uint8
    [rows, H], scales float32 [rows]): x ~ scale * (q1 + q2 / 16)."""
    x = _c(x_bf16, np.uint16)
    rows, H = x.shape
    q1 = np.empty((rows, H), dtype=np.uint8)
    q2 = np.empty((rows, H), dtype=np.uint8)
    sc = np.empty((rows,), dtype=np.float32)
    _load().oracle_quantize_fp8x2_rows(_p(x), rows, H, _p(q1), _p(q2), _p(sc))
    return q1, q2, sc


def _group(codes: np.ndarray, scales: np.ndarray) -> int:
    """Elements per scale of FP8 rows: one scale per row ([rows] scales) or per
    group of 128 ([rows, K/128] scales)."""
    rows, K = codes.shape
    if scales.size == rows:
        return K
    if scales.size == rows * (K // BLOCK) and K % BLOCK == 0:
        return BLOCK
    raise ValueError("scales must be [rows] or [rows, K/128]")


def quantize_fp8_groups(x_bf16: np.ndarray, group: int = BLOCK):
    """Block-scaled FP8 E4M3 quantization of bf16 rows, one scale per `group`
    consecutive elements -> (codes uint8 [rows, H], scales float32 [rows, H/group])."""
    x = _c(x_bf16, np.uint16)
    rows, H = x.shape
    if H % group:
        raise ValueError("H must be a multiple of the group")
    q = np.empty((rows, H), dtype=np.uint8)
    sc = np.empty((rows, H // group), dtype=np.float32)
    _load().oracle_quantize_fp8_groups(_p(x), rows, H, group, _p(q), _p(sc))
    return q, sc


def hidden_rows_fp8(aq: np.ndarray, a_scales: np.ndarray, w1: Weights, expert_of_row: np.ndarray,
                    I: int, activation: str = "silu", clamp: float = 0.0) -> np.ndarray:
    """hidden_rows on FP8 rows (decoded as code * the scale of its row, or of its
    group of 128 with [rows, H/128] scales), float64 [rows, I]."""
    aq = _c(aq, np.uint8)
    sc = _c(a_scales, np.float32)
    eor = _c(expert_of_row.astype(np.int32), np.int32)
    rows, H = aq.shape
    h = np.empty((rows, I), dtype=np.float64)
    _load().oracle_hidden_rows_fp8(_p(aq), _p(sc), _group(aq, sc), rows, H, I, w1.ref, _p(eor),
                                   ACTIVATIONS[activation], float(clamp), _p(h))
    return h


def out_rows_fp8(hq: np.ndarray, h_scales: np.ndarray, w2: Weights, expert_of_row: np.ndarray,
                 H: int) -> np.ndarray:
    """out_rows on FP8 rows (per-row or per-128-group scales), float64 [rows, H]."""
    hq = _c(hq, np.uint8)
    sc = _c(h_scales, np.float32)
    eor = _c(expert_of_row.astype(np.int32), np.int32)
    rows, I = hq.shape
    y = np.empty((rows, H), dtype=np.float64)
    _load().oracle_out_rows_fp8(_p(hq), _p(sc), _group(hq, sc), rows, I, H, w2.ref, _p(eor),
                                _p(y))
    return y


def hidden_rows_fp8x2(q1: np.ndarray, q2: np.ndarray, a_scales: np.ndarray, w1: Weights,
                      expert_of_row: np.ndarray, I: int, activation: str = "silu",
                      clamp: float = 0.0) -> np.ndarray:
    """hidden_rows on two-term FP8 rows, decoded to (q1 + q2 / 16) * scale."""
    a1, a2 = _c(q1, np.uint8), _c(q2, np.uint8)
    sc = _c(a_scales, np.float32)
    eor = _c(expert_of_row, np.int32)
    rows, H = a1.shape
    h = np.empty((rows, I), dtype=np.float64)
    _load().oracle_hidden_rows_fp8x2(_p(a1), _p(a2), _p(sc), rows, H, I, w1.ref, _p(eor),
                                     ACTIVATIONS[activation], float(clamp), _p(h))
    return h


def out_rows_fp8x2(q1: np.ndarray, q2: np.ndarray, h_scales: np.ndarray, w2: Weights,
                   expert_of_row: np.ndarray, H: int) -> np.ndarray:
    """out_rows on two-term FP8 rows, decoded to (q1 + q2 / 16) * scale."""
    a1, a2 = _c(q1, np.uint8), _c(q2, np.uint8)
    sc = _c(h_scales, np.float32)
    eor = _c(expert_of_row, np.int32)
    rows, I = a1.shape
    y = np.empty((rows, H), dtype=np.float64)
    _load().oracle_out_rows_fp8x2(_p(a1), _p(a2), _p(sc), rows, I, H, w2.ref, _p(eor), _p(y))
    return y


def hidden_rows(a_bf16: np.ndarray, w1: Weights, expert_of_row: np.ndarray, I: int,
                activation: str = "silu", clamp: float = 0.0) -> np.ndarray:
    """h[r] = act(W1g[e_r] a_r) * (W1u[e_r] a_r), float64 [rows, I]; act is
    "silu" or "gelu" (erf form); clamp > 0 limits the gate from above and the
    up value to [-clamp, clamp] first."""
    a = _c(a_bf16, np.uint16)
    eor = _c(expert_of_row.astype(np.int32), np.int32)
    rows, H = a.shape
    h = np.empty((rows, I), dtype=np.float64)
    _load().oracle_hidden_rows(_p(a), rows, H, I, w1.ref, _p(eor), ACTIVATIONS[activation],
                               float(clamp), _p(h))
    return h


def out_rows(h_bf16: np.ndarray, w2: Weights, expert_of_row: np.ndarray, H: int) -> np.ndarray:
    """y[r] = W2[e_r] h_r, float64 [rows, H]."""
    hb = _c(h_bf16, np.uint16)
    eor = _c(expert_of_row.astype(np.int32), np.int32)
    rows, I = hb.shape
    y = np.empty((rows, H), dtype=np.float64)
    _load().oracle_out_rows(_p(hb), rows, I, H, w2.ref, _p(eor), _p(y))
    return y


def finalize(y_perm_bf16: np.ndarray, weights: np.ndarray, pmap: np.ndarray, rsf_fin: float = 1.0,
             shared_bf16: Optional[np.ndarray] = None) -> np.ndarray:
    """out[t] = rsf_fin * sum_{map>=0} w * Y[map] + shared[t], float64 [T, H]."""
    y = _c(y_perm_bf16, np.uint16)
    w = _c(np.asarray(weights, dtype=np.float64), np.float64)
    pmap = _c(pmap, np.int32)
    shared = _c(shared_bf16, np.uint16)
    T, k = pmap.shape
    H = y.shape[1]
    out = np.empty((T, H), dtype=np.float64)
    _load().oracle_finalize(_p(y), _p(w), _p(pmap), T, k, H, rsf_fin, _p(shared), _p(out))
    return out


def finalize_add_rmsnorm(y_perm_bf16: np.ndarray, weights: np.ndarray, pmap: np.ndarray,
                         residual_bf16: np.ndarray, gamma_bf16: np.ndarray, eps: float,
                         rsf_fin: float = 1.0, shared_bf16: Optional[np.ndarray] = None):
    """Fused tail: (residual + finalize, RMSNorm of it times gamma), float64 [T, H] each."""
    y = _c(y_perm_bf16, np.uint16)
    w = _c(np.asarray(weights, dtype=np.float64), np.float64)
    pmap = _c(pmap, np.int32)
    shared = _c(shared_bf16, np.uint16)
    res = _c(residual_bf16, np.uint16)
    gamma = _c(gamma_bf16, np.uint16)
    T, k = pmap.shape
    H = y.shape[1]
    res_out = np.empty((T, H), dtype=np.float64)
    out = np.empty((T, H), dtype=np.float64)
    _load().oracle_finalize_add_rmsnorm(_p(y), _p(w), _p(pmap), T, k, H, rsf_fin, _p(shared),
                                        _p(res), _p(gamma), float(eps), _p(res_out), _p(out))
    return res_out, out


def moe_tokens(x_bf16: np.ndarray, logits: np.ndarray, w1: Weights, w2: Weights, I: int, k: int,
               score: int, renormalize: bool, rsf: float,
               expert_map: Optional[np.ndarray] = None, shared_I: int = 0,
               ws1: Optional[np.ndarray] = None, ws2: Optional[np.ndarray] = None,
               rsf_fin: float = 1.0, tokens: Optional[Sequence[int]] = None,
               activation: str = "silu", clamp: float = 0.0, weight_on_input: bool = False,
               fp8=False, a1_scale: Optional[float] = None,
               a2_scale: Optional[float] = None):
    """The whole layer for the listed tokens (all when None).  activation and
    clamp as for hidden_rows (every expert, the shared one included);
    weight_on_input: the routing weight scales the token before its expert
    MLP instead of the MLP's output (top_k = 1).  fp8: the routed experts see
    their input and hidden rows quantized per row to FP8 E4M3 (static
    a1_scale / a2_scale when given); fp8 "x2": quantized to two FP8 terms
    (quantize_fp8x2_rows); fp8 "block": quantized per group of 128 elements
    (quantize_fp8_groups), for block-scaled FP8 weights.

    Returns dict: out float64 [n, H], y_routes float64 [n, k, H] (unweighted
    per-route expert outputs, zero when not local), ids int32 [n, k],
    weights float64 [n, k], tokens int64 [n]."""
    x = _c(x_bf16, np.uint16)
    logits = _c(logits, np.float32)
    T, H = x.shape
    E = logits.shape[1]
    tok = np.arange(T, dtype=np.int64) if tokens is None else np.asarray(tokens, dtype=np.int64)
    tok = np.ascontiguousarray(tok)
    n = tok.shape[0]
    out = np.empty((n, H), dtype=np.float64)
    y = np.empty((n, k, H), dtype=np.float64)
    ids = np.empty((n, k), dtype=np.int32)
    w = np.empty((n, k), dtype=np.float64)
    expert_map = _c(expert_map, np.int32)
    ws1 = _c(ws1, np.uint16)
    ws2 = _c(ws2, np.uint16)
    s1 = None if a1_scale is None else np.array([a1_scale], dtype=np.float32)
    s2 = None if a2_scale is None else np.array([a2_scale], dtype=np.float32)
    _load().oracle_moe_tokens(_p(x), H, I, _p(logits), E, k, score, int(bool(renormalize)), rsf,
                              _p(expert_map), w1.ref, w2.ref, shared_I, _p(ws1), _p(ws2),
                              rsf_fin, ACTIVATIONS[activation], float(clamp),
                              int(bool(weight_on_input)),
                              {"x2": 2, "block": 3}.get(fp8, int(bool(fp8))) if isinstance(fp8, str)
                              else int(bool(fp8)),
                              _p(s1), _p(s2), _p(tok),
                              n, _p(out), _p(y), _p(ids), _p(w))
    return {"out": out, "y_routes": y, "ids": ids, "weights": w, "tokens": tok}
