"""Python binding of the C ABI in include/moe.h (argument marshalling only).

Every function has the name of the C call it wraps.  It checks what the MoE
output contract checks of its buffers (shape, dtype, device, contiguity),
allocates missing outputs with torch on the input's device, passes raw
pointers and the current HIP stream (or the given one) to the library and
raises ``MoeError`` on a non-zero status.  All arithmetic happens in the HIP
kernels; nothing here computes on the data.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from ._lib import MoeLayerOptionsC, MoeWeightsC, lib

SOFTMAX, SIGMOID = 0, 1
DTYPE_BF16, DTYPE_F32, DTYPE_MXFP4, DTYPE_FP8_E4M3, DTYPE_FP8_BLOCK = 0, 1, 2, 3, 4
QUANT_NONE, QUANT_FP8, QUANT_FP8X2, QUANT_FP8_BLOCK = 0, 1, 2, 3
ACT_SILU, ACT_GELU = 0, 1
_ACT_NAMES = {"silu": ACT_SILU, "gelu": ACT_GELU}


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def _check(status: int, name: str) -> None:
    if status != 0:
        L = lib()
        raise MoeError(status, f"{name}: {L.moe_status_string(status).decode()}: "
                               f"{L.moe_last_error().decode()}")


def _stream(stream) -> Optional[int]:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _hold(t: Optional[torch.Tensor], stream) -> None:
    """Keep a scratch tensor freed on return alive for work queued on `stream`
    (a caller's stream other than the current one)."""
    if t is not None and stream is not None:
        t.record_stream(stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _act(activation) -> int:
    return _ACT_NAMES[activation] if isinstance(activation, str) else int(activation)


def _quant(fp8) -> int:
    """act_quant of moe_layer_options: fp8 False (bf16 activations), True (FP8
    per token), "x2" (two-term FP8 of the bf16 activations, MXFP4 weights) or
    "block" (blockwise FP8 per 128-element group, block-scaled FP8 weights)."""
    if fp8 == "x2":
        return QUANT_FP8X2
    if fp8 == "block":
        return QUANT_FP8_BLOCK
    if fp8 in (False, True):
        return QUANT_FP8 if fp8 else QUANT_NONE
    raise ValueError(f"fp8 must be False, True, 'x2' or 'block' (got {fp8!r})")


def _options(activation=ACT_SILU, activation_clamp: Optional[float] = None,
             apply_router_weight_on_input: bool = False, chunk_tokens: int = 0,
             batched_max_tokens: int = 0, fp8=False,
             a1_scale: Optional[torch.Tensor] = None, a2_scale: Optional[torch.Tensor] = None):
    """moe_layer_options by reference (None when every option is its default)."""
    act = _act(activation)
    clamp = 0.0 if activation_clamp is None else float(activation_clamp)
    if (act == ACT_SILU and clamp == 0.0 and not apply_router_weight_on_input
            and not chunk_tokens and not batched_max_tokens and not fp8
            and a1_scale is None and a2_scale is None):
        return None
    for name, t in (("a1_scale", a1_scale), ("a2_scale", a2_scale)):
        if t is not None:
            _need(t, name, torch.float32)
            if t.numel() != 1:
                raise ValueError(f"{name} must hold one float32")
    return ctypes.byref(MoeLayerOptionsC(act, clamp, int(bool(apply_router_weight_on_input)),
                                         int(chunk_tokens), int(batched_max_tokens),
                                         _quant(fp8), _ptr(a1_scale),
                                         _ptr(a2_scale)))


def _weights_arg(expert_weights: Optional[torch.Tensor], T: int, k: int, dev):
    """(pointer, dtype tag) of finalize's weights; None means unit weights."""
    if expert_weights is None:
        return None, DTYPE_F32
    if expert_weights.dtype == torch.float32:
        wdt = DTYPE_F32
    elif expert_weights.dtype == torch.bfloat16:
        wdt = DTYPE_BF16
    else:
        raise TypeError("expert_weights must be float32 or bfloat16")
    _need(expert_weights, "expert_weights", expert_weights.dtype, device=dev)
    if expert_weights.numel() != T * k:
        raise ValueError(f"expert_weights must have T * k = {T * k} elements")
    return expert_weights.data_ptr(), wdt


def _need(t: torch.Tensor, name: str, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    return t


class Weights:
    """Expert weights of one GEMM: bf16 [E_l, N, K]; MXFP4 packed uint8
    [E_l, N, K/2] with uint8 E8M0 scales [E_l, N, K/32]; FP8 E4M3 codes
    (uint8 or float8_e4m3fn) [E_l, N, K] with float32 scales [E_l, N]; or
    block-scaled FP8 codes [E_l, N, K] with float32 scales [E_l, N/128, K/128]
    (one per 128 x 128 block)."""

    def __init__(self, data: torch.Tensor, scales: Optional[torch.Tensor] = None):
        if data.dtype == torch.float8_e4m3fn:
            data = data.view(torch.uint8)
        if scales is None:
            _need(data, "weights", torch.bfloat16)
            self.dtype = DTYPE_BF16
        elif scales.dtype == torch.float32 and scales.dim() == 3:
            _need(data, "weights", torch.uint8)
            if data.dim() != 3 or data.shape[1] % 128 or data.shape[2] % 128:
                raise ValueError("block-scaled FP8 weights need N and K multiples of 128")
            _need(scales, "scales", torch.float32,
                  (data.shape[0], data.shape[1] // 128, data.shape[2] // 128), data.device)
            self.dtype = DTYPE_FP8_BLOCK
        elif scales.dtype == torch.float32:
            _need(data, "weights", torch.uint8)
            _need(scales, "scales", torch.float32, tuple(data.shape[:2]), data.device)
            self.dtype = DTYPE_FP8_E4M3
        else:
            _need(data, "weights", torch.uint8)
            _need(scales, "scales", torch.uint8, device=data.device)
            self.dtype = DTYPE_MXFP4
        if data.dim() != 3:
            raise ValueError("weights must be rank-3 [E_l, N, K(/2)]")
        self.data, self.scales = data, scales
        self.c = MoeWeightsC(self.dtype, data.data_ptr(), _ptr(scales))

    @property
    def E_l(self) -> int:
        return self.data.shape[0]

    @property
    def N(self) -> int:
        return self.data.shape[1]

    @property
    def K(self) -> int:
        k = self.data.shape[2]
        return k * 2 if self.dtype == DTYPE_MXFP4 else k

    def ref(self):
        return ctypes.byref(self.c)


def moe_permuted_rows(T: int, k: int) -> int:
    return int(lib().moe_permuted_rows(T, k))


def moe_workspace_size(T: int, k: int, E: int, E_l: int, H: int, I: int,
                       w_dtype: int = DTYPE_BF16, shared_I: int = 0, chunk_tokens: int = 0,
                       batched_max_tokens: int = 0, fp8=False) -> int:
    """Workspace bytes of the fused calls (the shared expert's included)."""
    n = ctypes.c_size_t(0)
    opts = _options(chunk_tokens=chunk_tokens, batched_max_tokens=batched_max_tokens, fp8=fp8)
    _check(lib().moe_workspace_size(T, k, E, E_l, H, I, w_dtype, shared_I, opts, ctypes.byref(n)),
           "moe_workspace_size")
    return int(n.value)


def moe_shared_workspace_size(T: int, H: int, shared_I: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_shared_workspace_size(T, H, shared_I, ctypes.byref(n)),
           "moe_shared_workspace_size")
    return int(n.value)


def moe_route_topk(logits: torch.Tensor, k: int, score_fn: int = SOFTMAX, renormalize: bool = True,
                   rsf: float = 1.0, topk_ids: Optional[torch.Tensor] = None,
                   topk_weights: Optional[torch.Tensor] = None, stream=None):
    """-> (topk_ids int32 [T, k], topk_weights float32 [T, k])."""
    _need(logits, "logits", torch.float32)
    if logits.dim() != 2:
        raise ValueError("logits must be rank-2 [T, E]")
    T, E = logits.shape
    dev = logits.device
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_weights is None:
        topk_weights = torch.empty((T, k), dtype=torch.float32, device=dev)
    _need(topk_ids, "topk_ids", torch.int32, (T, k), dev)
    _need(topk_weights, "topk_weights", torch.float32, (T, k), dev)
    _check(lib().moe_route_topk(logits.data_ptr(), T, E, k, score_fn, int(bool(renormalize)),
                                float(rsf), topk_ids.data_ptr(), topk_weights.data_ptr(),
                                _stream(stream)), "moe_route_topk")
    return topk_ids, topk_weights


def moe_route_permute(logits: torch.Tensor, k: int, score_fn: int = SOFTMAX,
                      renormalize: bool = True, rsf: float = 1.0, E_l: Optional[int] = None,
                      expert_map: Optional[torch.Tensor] = None, R_pad: Optional[int] = None,
                      topk_ids: Optional[torch.Tensor] = None,
                      topk_weights: Optional[torch.Tensor] = None,
                      map: Optional[torch.Tensor] = None, offsets: Optional[torch.Tensor] = None,
                      inv: Optional[torch.Tensor] = None, want_inv: bool = True, stream=None):
    """Router and permute map in one call (one kernel for T <= 16).
    -> dict(topk_ids, topk_weights, map, offsets, inv or None, R_pad)."""
    _need(logits, "logits", torch.float32)
    if logits.dim() != 2:
        raise ValueError("logits must be rank-2 [T, E]")
    T, E = logits.shape
    dev = logits.device
    E_l = E if E_l is None else E_l
    if expert_map is not None:
        _need(expert_map, "expert_map", torch.int32, (E,), dev)
    R_pad = moe_permuted_rows(T, k) if R_pad is None else R_pad
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_weights is None:
        topk_weights = torch.empty((T, k), dtype=torch.float32, device=dev)
    if map is None:
        map = torch.empty((T, k), dtype=torch.int32, device=dev)
    if offsets is None:
        offsets = torch.empty((E_l + 1,), dtype=torch.int32, device=dev)
    if inv is None and want_inv and R_pad > 0:
        inv = torch.empty((R_pad,), dtype=torch.int32, device=dev)
    _need(topk_ids, "topk_ids", torch.int32, (T, k), dev)
    _need(topk_weights, "topk_weights", torch.float32, (T, k), dev)
    _need(map, "map", torch.int32, (T, k), dev)
    _need(offsets, "offsets", torch.int32, (E_l + 1,), dev)
    if inv is not None:
        _need(inv, "inv", torch.int32, (R_pad,), dev)
    _check(lib().moe_route_permute(logits.data_ptr(), T, E, k, score_fn, int(bool(renormalize)),
                                   float(rsf), _ptr(expert_map), E_l, R_pad, topk_ids.data_ptr(),
                                   topk_weights.data_ptr(), map.data_ptr(), offsets.data_ptr(),
                                   _ptr(inv), _stream(stream)), "moe_route_permute")
    return {"topk_ids": topk_ids, "topk_weights": topk_weights, "map": map, "offsets": offsets,
            "inv": inv, "R_pad": R_pad}


def moe_permute(topk_ids: torch.Tensor, E: int, E_l: Optional[int] = None,
                expert_map: Optional[torch.Tensor] = None, x: Optional[torch.Tensor] = None,
                R_pad: Optional[int] = None, map: Optional[torch.Tensor] = None,
                offsets: Optional[torch.Tensor] = None, inv: Optional[torch.Tensor] = None,
                x_perm: Optional[torch.Tensor] = None, want_inv: bool = True,
                x_weights: Optional[torch.Tensor] = None, stream=None):
    """-> dict(map [T,k] int32, offsets [E_l+1] int32, inv [R_pad] int32 or None,
    x_perm [R_pad, H] bf16 or None, R_pad).  x_weights (fp32 [T, k]): each
    gathered row is scaled by its routing weight (apply_router_weight_on_input)."""
    _need(topk_ids, "topk_ids", torch.int32)
    T, k = topk_ids.shape
    dev = topk_ids.device
    E_l = E if E_l is None else E_l
    if expert_map is not None:
        _need(expert_map, "expert_map", torch.int32, (E,), dev)
    R_pad = moe_permuted_rows(T, k) if R_pad is None else R_pad
    H = 0
    if x is not None:
        _need(x, "x", torch.bfloat16, device=dev)
        if x.dim() != 2 or x.shape[0] != T:
            raise ValueError("x must be [T, H]")
        H = x.shape[1]
        if x_perm is None:
            x_perm = torch.empty((R_pad, H), dtype=torch.bfloat16, device=dev)
        _need(x_perm, "x_perm", torch.bfloat16, (R_pad, H), dev)
    if map is None:
        map = torch.empty((T, k), dtype=torch.int32, device=dev)
    if offsets is None:
        offsets = torch.empty((E_l + 1,), dtype=torch.int32, device=dev)
    if inv is None and want_inv and R_pad > 0:
        inv = torch.empty((R_pad,), dtype=torch.int32, device=dev)
    _need(map, "map", torch.int32, (T, k), dev)
    _need(offsets, "offsets", torch.int32, (E_l + 1,), dev)
    if inv is not None:
        _need(inv, "inv", torch.int32, (R_pad,), dev)
    if x_weights is not None:
        _need(x_weights, "x_weights", torch.float32, (T, k), dev)
    _check(lib().moe_permute(topk_ids.data_ptr(), _ptr(expert_map), T, k, E, E_l, _ptr(x), H,
                             R_pad, map.data_ptr(), offsets.data_ptr(), _ptr(inv), _ptr(x_perm),
                             _ptr(x_weights), None, 0, _stream(stream)), "moe_permute")
    return {"map": map, "offsets": offsets, "inv": inv, "x_perm": x_perm, "R_pad": R_pad}


def moe_quantize_fp8(x: torch.Tensor, static_scale: Optional[torch.Tensor] = None,
                     row_weights: Optional[torch.Tensor] = None, q: Optional[torch.Tensor] = None,
                     scales: Optional[torch.Tensor] = None, row_count: Optional[torch.Tensor] = None,
                     stream=None):
    """Per-row FP8 E4M3 quantization of bf16 rows -> (codes uint8 [rows, H],
    scales float32 [rows]).  row_count: an int32 device scalar (say offsets[E_l:])
    limiting the rows quantized."""
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be [rows, H]")
    rows, H = x.shape
    dev = x.device
    if q is None:
        q = torch.empty((rows, H), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows,), dtype=torch.float32, device=dev)
    _need(q, "q", torch.uint8, (rows, H), dev)
    _need(scales, "scales", torch.float32, (rows,), dev)
    if static_scale is not None:
        _need(static_scale, "static_scale", torch.float32, device=dev)
    if row_weights is not None:
        _need(row_weights, "row_weights", torch.float32, device=dev)
        if row_weights.numel() != rows:
            raise ValueError("row_weights must hold one float32 per row")
    if row_count is not None:
        _need(row_count, "row_count", torch.int32, device=dev)
    _check(lib().moe_quantize_fp8(x.data_ptr(), rows, H, _ptr(static_scale), _ptr(row_weights),
                                  _ptr(row_count), q.data_ptr(), scales.data_ptr(),
                                  _stream(stream)),
           "moe_quantize_fp8")
    return q, scales


def moe_permute_fp8(topk_ids: torch.Tensor, E: int, xq: torch.Tensor, x_scales: torch.Tensor,
                    E_l: Optional[int] = None, expert_map: Optional[torch.Tensor] = None,
                    R_pad: Optional[int] = None, map: Optional[torch.Tensor] = None,
                    offsets: Optional[torch.Tensor] = None, inv: Optional[torch.Tensor] = None,
                    xq_perm: Optional[torch.Tensor] = None,
                    xq_perm_scales: Optional[torch.Tensor] = None, want_inv: bool = True,
                    stream=None):
    """moe_permute on FP8 rows -> dict(map, offsets, inv, xq_perm uint8 [R_pad, H],
    xq_perm_scales float32 [R_pad], R_pad)."""
    _need(topk_ids, "topk_ids", torch.int32)
    T, k = topk_ids.shape
    dev = topk_ids.device
    E_l = E if E_l is None else E_l
    _need(xq, "xq", torch.uint8, device=dev)
    if xq.dim() != 2 or xq.shape[0] != T:
        raise ValueError("xq must be [T, H]")
    H = xq.shape[1]
    _need(x_scales, "x_scales", torch.float32, (T,), dev)
    if expert_map is not None:
        _need(expert_map, "expert_map", torch.int32, (E,), dev)
    R_pad = moe_permuted_rows(T, k) if R_pad is None else R_pad
    if map is None:
        map = torch.empty((T, k), dtype=torch.int32, device=dev)
    if offsets is None:
        offsets = torch.empty((E_l + 1,), dtype=torch.int32, device=dev)
    if inv is None and want_inv and R_pad > 0:
        inv = torch.empty((R_pad,), dtype=torch.int32, device=dev)
    if xq_perm is None:
        xq_perm = torch.empty((R_pad, H), dtype=torch.uint8, device=dev)
    if xq_perm_scales is None:
        xq_perm_scales = torch.empty((R_pad,), dtype=torch.float32, device=dev)
    _need(map, "map", torch.int32, (T, k), dev)
    _need(offsets, "offsets", torch.int32, (E_l + 1,), dev)
    _need(xq_perm, "xq_perm", torch.uint8, (R_pad, H), dev)
    _need(xq_perm_scales, "xq_perm_scales", torch.float32, (R_pad,), dev)
    _check(lib().moe_permute_fp8(topk_ids.data_ptr(), _ptr(expert_map), T, k, E, E_l,
                                 xq.data_ptr(), x_scales.data_ptr(), H, R_pad, map.data_ptr(),
                                 offsets.data_ptr(), _ptr(inv), xq_perm.data_ptr(),
                                 xq_perm_scales.data_ptr(), _stream(stream)), "moe_permute_fp8")
    return {"map": map, "offsets": offsets, "inv": inv, "xq_perm": xq_perm,
            "xq_perm_scales": xq_perm_scales, "R_pad": R_pad}


def moe_grouped_gemm1_act_fp8(a_perm: torch.Tensor, a_scales: torch.Tensor,
                              offsets: torch.Tensor, w1: Weights, I: int,
                              h: Optional[torch.Tensor] = None, activation=ACT_SILU,
                              activation_clamp: Optional[float] = None, stream=None,
                              split: bool = True,
                              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """GEMM1 + activation on FP8 rows and FP8 weights -> bf16 [R_pad, I]."""
    _need(a_perm, "a_perm", torch.uint8)
    R_pad, H = a_perm.shape
    dev = a_perm.device
    _need(a_scales, "a_scales", torch.float32, (R_pad,), dev)
    _need(offsets, "offsets", torch.int32, (w1.E_l + 1,), dev)
    if w1.N != 2 * I or w1.K != H:
        raise ValueError(f"w1 must be [E_l, 2I={2 * I}, H={H}]")
    if h is None:
        h = torch.empty((R_pad, I), dtype=torch.bfloat16, device=dev)
    _need(h, "h", torch.bfloat16, (R_pad, I), dev)
    ws, ws_bytes, _keep = _gemm_workspace(R_pad, I, True, split, dev, stream, workspace)
    _check(lib().moe_grouped_gemm1_act_fp8(
        a_perm.data_ptr(), a_scales.data_ptr(), offsets.data_ptr(), w1.E_l, R_pad, H, I, w1.ref(),
        _act(activation), 0.0 if activation_clamp is None else float(activation_clamp),
        h.data_ptr(), ws, ws_bytes, _stream(stream)), "moe_grouped_gemm1_act_fp8")
    return h


def moe_grouped_gemm2_fp8(h_perm: torch.Tensor, h_scales: torch.Tensor, offsets: torch.Tensor,
                          w2: Weights, H: int, y: Optional[torch.Tensor] = None, stream=None,
                          split: bool = True,
                          workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """GEMM2 on FP8 rows and FP8 weights -> bf16 [R_pad, H]."""
    _need(h_perm, "h_perm", torch.uint8)
    R_pad, I = h_perm.shape
    dev = h_perm.device
    _need(h_scales, "h_scales", torch.float32, (R_pad,), dev)
    _need(offsets, "offsets", torch.int32, (w2.E_l + 1,), dev)
    if w2.N != H or w2.K != I:
        raise ValueError(f"w2 must be [E_l, H={H}, I={I}]")
    if y is None:
        y = torch.empty((R_pad, H), dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, (R_pad, H), dev)
    ws, ws_bytes, _keep = _gemm_workspace(R_pad, H, False, split, dev, stream, workspace)
    _check(lib().moe_grouped_gemm2_fp8(
        h_perm.data_ptr(), h_scales.data_ptr(), offsets.data_ptr(), w2.E_l, R_pad, I, H, w2.ref(),
        y.data_ptr(), ws, ws_bytes, _stream(stream)), "moe_grouped_gemm2_fp8")
    return y


def moe_grouped_gemm1_act_fp8_gathered(xq: torch.Tensor, x_scales: torch.Tensor,
                                       inv: torch.Tensor, k: int, offsets: torch.Tensor,
                                       w1: Weights, I: int, terms: int = 1,
                                       h: Optional[torch.Tensor] = None, activation=ACT_SILU,
                                       activation_clamp: Optional[float] = None, stream=None,
                                       split: bool = True,
                                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """FP8 GEMM1 on rows read from the quantized tokens: permuted row r is
    xq[inv[r] // k] with scale x_scales[inv[r] // k] (xq [T, H * terms]) -> bf16
    [R_pad, I], R_pad = inv's length."""
    _need(xq, "xq", torch.uint8)
    if xq.dim() != 2 or terms not in (1, 2):
        raise ValueError("xq must be [T, H * terms], terms 1 or 2")
    T = xq.shape[0]
    H = xq.shape[1] // terms
    dev = xq.device
    _need(x_scales, "x_scales", torch.float32, (T,), dev)
    _need(inv, "inv", torch.int32, device=dev)
    R_pad = inv.numel()
    _need(offsets, "offsets", torch.int32, (w1.E_l + 1,), dev)
    if w1.N != 2 * I or w1.K != H:
        raise ValueError(f"w1 must be [E_l, 2I={2 * I}, H={H}]")
    if h is None:
        h = torch.empty((R_pad, I), dtype=torch.bfloat16, device=dev)
    _need(h, "h", torch.bfloat16, (R_pad, I), dev)
    ws, ws_bytes, _keep = _gemm_workspace(R_pad, I, True, split, dev, stream, workspace)
    _check(lib().moe_grouped_gemm1_act_fp8_gathered(
        xq.data_ptr(), x_scales.data_ptr(), terms, inv.data_ptr(), T, k, offsets.data_ptr(),
        w1.E_l, R_pad, H, I, w1.ref(), _act(activation),
        0.0 if activation_clamp is None else float(activation_clamp), h.data_ptr(), ws, ws_bytes,
        _stream(stream)), "moe_grouped_gemm1_act_fp8_gathered")
    return h


def moe_quantize_fp8_blockwise(x: torch.Tensor, row_count: Optional[torch.Tensor] = None,
                               q: Optional[torch.Tensor] = None,
                               scales: Optional[torch.Tensor] = None, stream=None):
    """Blockwise FP8 E4M3 quantization of bf16 rows, one scale per row and group
    of 128 elements -> (codes uint8 [rows, H], scales float32 [H/128, ld]
    group-major, ld = rows unless `scales` gives a wider one)."""
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be [rows, H]")
    rows, H = x.shape
    dev = x.device
    if q is None:
        q = torch.empty((rows, H), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((H // 128, rows), dtype=torch.float32, device=dev)
    _need(q, "q", torch.uint8, (rows, H), dev)
    _need(scales, "scales", torch.float32, device=dev)
    if scales.dim() != 2 or scales.shape[0] != H // 128 or scales.shape[1] < rows:
        raise ValueError("scales must be [H/128, ld >= rows]")
    if row_count is not None:
        _need(row_count, "row_count", torch.int32, device=dev)
    _check(lib().moe_quantize_fp8_blockwise(x.data_ptr(), rows, H, _ptr(row_count), q.data_ptr(),
                                            scales.data_ptr(), scales.shape[1], _stream(stream)),
           "moe_quantize_fp8_blockwise")
    return q, scales


def moe_permute_fp8_blockwise(topk_ids: torch.Tensor, E: int, xq: torch.Tensor,
                              x_scales: torch.Tensor, E_l: Optional[int] = None,
                              expert_map: Optional[torch.Tensor] = None,
                              R_pad: Optional[int] = None, map: Optional[torch.Tensor] = None,
                              offsets: Optional[torch.Tensor] = None,
                              inv: Optional[torch.Tensor] = None,
                              xq_perm: Optional[torch.Tensor] = None,
                              xq_perm_scales: Optional[torch.Tensor] = None,
                              want_inv: bool = True, stream=None):
    """moe_permute on blockwise FP8 rows -> dict(map, offsets, inv, xq_perm uint8
    [R_pad, H], xq_perm_scales float32 [H/128, R_pad], R_pad)."""
    _need(topk_ids, "topk_ids", torch.int32)
    T, k = topk_ids.shape
    dev = topk_ids.device
    E_l = E if E_l is None else E_l
    _need(xq, "xq", torch.uint8, device=dev)
    if xq.dim() != 2 or xq.shape[0] != T:
        raise ValueError("xq must be [T, H]")
    H = xq.shape[1]
    _need(x_scales, "x_scales", torch.float32, (H // 128, T), dev)
    if expert_map is not None:
        _need(expert_map, "expert_map", torch.int32, (E,), dev)
    R_pad = moe_permuted_rows(T, k) if R_pad is None else R_pad
    if map is None:
        map = torch.empty((T, k), dtype=torch.int32, device=dev)
    if offsets is None:
        offsets = torch.empty((E_l + 1,), dtype=torch.int32, device=dev)
    if inv is None and want_inv and R_pad > 0:
        inv = torch.empty((R_pad,), dtype=torch.int32, device=dev)
    if xq_perm is None:
        xq_perm = torch.empty((R_pad, H), dtype=torch.uint8, device=dev)
    if xq_perm_scales is None:
        xq_perm_scales = torch.empty((H // 128, R_pad), dtype=torch.float32, device=dev)
    _need(map, "map", torch.int32, (T, k), dev)
    _need(offsets, "offsets", torch.int32, (E_l + 1,), dev)
    _need(xq_perm, "xq_perm", torch.uint8, (R_pad, H), dev)
    _need(xq_perm_scales, "xq_perm_scales", torch.float32, (H // 128, R_pad), dev)
    _check(lib().moe_permute_fp8_blockwise(topk_ids.data_ptr(), _ptr(expert_map), T, k, E, E_l,
                                           xq.data_ptr(), x_scales.data_ptr(), H, R_pad,
                                           map.data_ptr(), offsets.data_ptr(), _ptr(inv),
                                           xq_perm.data_ptr(), xq_perm_scales.data_ptr(),
                                           _stream(stream)), "moe_permute_fp8_blockwise")
    return {"map": map, "offsets": offsets, "inv": inv, "xq_perm": xq_perm,
            "xq_perm_scales": xq_perm_scales, "R_pad": R_pad}


def moe_grouped_gemm1_act_fp8_blockwise(a_perm: torch.Tensor, a_scales: torch.Tensor,
                                        offsets: torch.Tensor, w1: Weights, I: int,
                                        h: Optional[torch.Tensor] = None, activation=ACT_SILU,
                                        activation_clamp: Optional[float] = None, stream=None,
                                        split: bool = True,
                                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """GEMM1 + activation on blockwise FP8 rows (scales [H/128, R_pad]) and
    block-scaled FP8 weights -> bf16 [R_pad, I]."""
    _need(a_perm, "a_perm", torch.uint8)
    R_pad, H = a_perm.shape
    dev = a_perm.device
    _need(a_scales, "a_scales", torch.float32, (H // 128, R_pad), dev)
    _need(offsets, "offsets", torch.int32, (w1.E_l + 1,), dev)
    if w1.N != 2 * I or w1.K != H:
        raise ValueError(f"w1 must be [E_l, 2I={2 * I}, H={H}]")
    if h is None:
        h = torch.empty((R_pad, I), dtype=torch.bfloat16, device=dev)
    _need(h, "h", torch.bfloat16, (R_pad, I), dev)
    ws, ws_bytes, _keep = _gemm_workspace(R_pad, I, True, split, dev, stream, workspace)
    _check(lib().moe_grouped_gemm1_act_fp8_blockwise(
        a_perm.data_ptr(), a_scales.data_ptr(), offsets.data_ptr(), w1.E_l, R_pad, H, I, w1.ref(),
        _act(activation), 0.0 if activation_clamp is None else float(activation_clamp),
        h.data_ptr(), ws, ws_bytes, _stream(stream)), "moe_grouped_gemm1_act_fp8_blockwise")
    return h


def moe_grouped_gemm2_fp8_blockwise(h_perm: torch.Tensor, h_scales: torch.Tensor,
                                    offsets: torch.Tensor, w2: Weights, H: int,
                                    y: Optional[torch.Tensor] = None, stream=None,
                                    split: bool = True,
                                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """GEMM2 on blockwise FP8 rows (scales [I/128, R_pad]) and block-scaled FP8
    weights -> bf16 [R_pad, H]."""
    _need(h_perm, "h_perm", torch.uint8)
    R_pad, I = h_perm.shape
    dev = h_perm.device
    _need(h_scales, "h_scales", torch.float32, (I // 128, R_pad), dev)
    _need(offsets, "offsets", torch.int32, (w2.E_l + 1,), dev)
    if w2.N != H or w2.K != I:
        raise ValueError(f"w2 must be [E_l, H={H}, I={I}]")
    if y is None:
        y = torch.empty((R_pad, H), dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, (R_pad, H), dev)
    ws, ws_bytes, _keep = _gemm_workspace(R_pad, H, False, split, dev, stream, workspace)
    _check(lib().moe_grouped_gemm2_fp8_blockwise(
        h_perm.data_ptr(), h_scales.data_ptr(), offsets.data_ptr(), w2.E_l, R_pad, I, H, w2.ref(),
        y.data_ptr(), ws, ws_bytes, _stream(stream)), "moe_grouped_gemm2_fp8_blockwise")
    return y


def moe_quantize_fp8x2(x: torch.Tensor, row_weights: Optional[torch.Tensor] = None,
                       q: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                       row_count: Optional[torch.Tensor] = None, stream=None):
    """Two-term FP8 E4M3 quantization of bf16 rows -> (codes uint8 [rows, 2H]:
    per 64 k the first term's 64 codes, then the second's; scales float32
    [rows]), x ~ scale * (q1 + q2 / 16)."""
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be [rows, H]")
    rows, H = x.shape
    dev = x.device
    if q is None:
        q = torch.empty((rows, 2 * H), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows,), dtype=torch.float32, device=dev)
    _need(q, "q", torch.uint8, (rows, 2 * H), dev)
    _need(scales, "scales", torch.float32, (rows,), dev)
    if row_weights is not None:
        _need(row_weights, "row_weights", torch.float32, device=dev)
        if row_weights.numel() != rows:
            raise ValueError("row_weights must hold one float32 per row")
    if row_count is not None:
        _need(row_count, "row_count", torch.int32, device=dev)
    _check(lib().moe_quantize_fp8x2(x.data_ptr(), rows, H, _ptr(row_weights), _ptr(row_count),
                                    q.data_ptr(), scales.data_ptr(), _stream(stream)),
           "moe_quantize_fp8x2")
    return q, scales


def moe_grouped_gemm1_act_fp8x2(a_perm: torch.Tensor, a_scales: torch.Tensor,
                                offsets: torch.Tensor, w1: Weights, I: int,
                                h: Optional[torch.Tensor] = None, activation=ACT_SILU,
                                activation_clamp: Optional[float] = None, stream=None,
                                split: bool = True,
                                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """GEMM1 + activation on two-term FP8 rows [R_pad, 2H] and MXFP4 weights -> bf16 [R_pad, I]."""
    _need(a_perm, "a_perm", torch.uint8)
    R_pad, H2 = a_perm.shape
    H = H2 // 2
    dev = a_perm.device
    _need(a_scales, "a_scales", torch.float32, (R_pad,), dev)
    _need(offsets, "offsets", torch.int32, (w1.E_l + 1,), dev)
    if H2 % 2 or w1.N != 2 * I or w1.K != H:
        raise ValueError(f"w1 must be [E_l, 2I={2 * I}, H={H}] for rows of 2H bytes")
    if h is None:
        h = torch.empty((R_pad, I), dtype=torch.bfloat16, device=dev)
    _need(h, "h", torch.bfloat16, (R_pad, I), dev)
    ws, ws_bytes, _keep = _gemm_workspace(R_pad, I, True, split, dev, stream, workspace)
    _check(lib().moe_grouped_gemm1_act_fp8x2(
        a_perm.data_ptr(), a_scales.data_ptr(), offsets.data_ptr(), w1.E_l, R_pad, H, I, w1.ref(),
        _act(activation), 0.0 if activation_clamp is None else float(activation_clamp),
        h.data_ptr(), ws, ws_bytes, _stream(stream)), "moe_grouped_gemm1_act_fp8x2")
    return h


def moe_grouped_gemm2_fp8x2(h_perm: torch.Tensor, h_scales: torch.Tensor, offsets: torch.Tensor,
                            w2: Weights, H: int, y: Optional[torch.Tensor] = None, stream=None,
                            split: bool = True,
                            workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """GEMM2 on two-term FP8 rows [R_pad, 2I] and MXFP4 weights -> bf16 [R_pad, H]."""
    _need(h_perm, "h_perm", torch.uint8)
    R_pad, I2 = h_perm.shape
    I = I2 // 2
    dev = h_perm.device
    _need(h_scales, "h_scales", torch.float32, (R_pad,), dev)
    _need(offsets, "offsets", torch.int32, (w2.E_l + 1,), dev)
    if I2 % 2 or w2.N != H or w2.K != I:
        raise ValueError(f"w2 must be [E_l, H={H}, I={I}] for rows of 2I bytes")
    if y is None:
        y = torch.empty((R_pad, H), dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, (R_pad, H), dev)
    ws, ws_bytes, _keep = _gemm_workspace(R_pad, H, False, split, dev, stream, workspace)
    _check(lib().moe_grouped_gemm2_fp8x2(
        h_perm.data_ptr(), h_scales.data_ptr(), offsets.data_ptr(), w2.E_l, R_pad, I, H, w2.ref(),
        y.data_ptr(), ws, ws_bytes, _stream(stream)), "moe_grouped_gemm2_fp8x2")
    return y


def moe_permute_batched(topk_ids: torch.Tensor, E: int, max_tokens: int, E_l: Optional[int] = None,
                        expert_map: Optional[torch.Tensor] = None,
                        x: Optional[torch.Tensor] = None, map: Optional[torch.Tensor] = None,
                        expert_num_tokens: Optional[torch.Tensor] = None,
                        x_batched: Optional[torch.Tensor] = None,
                        x_weights: Optional[torch.Tensor] = None, stream=None):
    """Batched experts format -> dict(map [T,k] int32, expert_num_tokens [E_l]
    int32, x_batched [E_l, max_tokens, H] bf16 or None)."""
    _need(topk_ids, "topk_ids", torch.int32)
    T, k = topk_ids.shape
    dev = topk_ids.device
    E_l = E if E_l is None else E_l
    if expert_map is not None:
        _need(expert_map, "expert_map", torch.int32, (E,), dev)
    H = 0
    if x is not None:
        _need(x, "x", torch.bfloat16, device=dev)
        if x.dim() != 2 or x.shape[0] != T:
            raise ValueError("x must be [T, H]")
        H = x.shape[1]
        if x_batched is None:
            x_batched = torch.empty((E_l, max_tokens, H), dtype=torch.bfloat16, device=dev)
        _need(x_batched, "x_batched", torch.bfloat16, (E_l, max_tokens, H), dev)
    if map is None:
        map = torch.empty((T, k), dtype=torch.int32, device=dev)
    if expert_num_tokens is None:
        expert_num_tokens = torch.empty((E_l,), dtype=torch.int32, device=dev)
    _need(map, "map", torch.int32, (T, k), dev)
    _need(expert_num_tokens, "expert_num_tokens", torch.int32, (E_l,), dev)
    if x_weights is not None:
        _need(x_weights, "x_weights", torch.float32, (T, k), dev)
    _check(lib().moe_permute_batched(topk_ids.data_ptr(), _ptr(expert_map), T, k, E, E_l, _ptr(x),
                                     H, max_tokens, map.data_ptr(), expert_num_tokens.data_ptr(),
                                     _ptr(x_batched), _ptr(x_weights), _stream(stream)),
           "moe_permute_batched")
    return {"map": map, "expert_num_tokens": expert_num_tokens, "x_batched": x_batched}


def _batched_in(a: torch.Tensor, name: str):
    _need(a, name, torch.bfloat16)
    if a.dim() != 3:
        raise ValueError(f"{name} must be [E_l, max_tokens, K]")
    return a.shape


def moe_grouped_gemm1_act_batched(a_batched: torch.Tensor, expert_num_tokens: torch.Tensor,
                                  w1: Weights, I: int, h_batched: Optional[torch.Tensor] = None,
                                  activation=ACT_SILU, activation_clamp: Optional[float] = None,
                                  max_rows: int = 0, stream=None, split: bool = True,
                                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """GEMM1 + activation in the batched experts format -> bf16 [E_l, max_tokens, I]."""
    E_l, M, H = _batched_in(a_batched, "a_batched")
    dev = a_batched.device
    _need(expert_num_tokens, "expert_num_tokens", torch.int32, (E_l,), dev)
    if w1.E_l != E_l or w1.N != 2 * I or w1.K != H:
        raise ValueError(f"w1 must be [E_l={E_l}, 2I={2 * I}, H={H}]")
    if h_batched is None:
        h_batched = torch.empty((E_l, M, I), dtype=torch.bfloat16, device=dev)
    _need(h_batched, "h_batched", torch.bfloat16, (E_l, M, I), dev)
    ws, ws_bytes, _keep = _gemm_workspace(E_l * M, I, True, split, dev, stream, workspace)
    _check(lib().moe_grouped_gemm1_act_batched(
        a_batched.data_ptr(), expert_num_tokens.data_ptr(), E_l, M, max_rows, H, I, w1.ref(),
        _act(activation), 0.0 if activation_clamp is None else float(activation_clamp),
        h_batched.data_ptr(), ws, ws_bytes, _stream(stream)), "moe_grouped_gemm1_act_batched")
    return h_batched


def moe_grouped_gemm2_batched(h_batched: torch.Tensor, expert_num_tokens: torch.Tensor,
                              w2: Weights, H: int, y_batched: Optional[torch.Tensor] = None,
                              max_rows: int = 0, stream=None, split: bool = True,
                              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """GEMM2 in the batched experts format -> bf16 [E_l, max_tokens, H]."""
    E_l, M, I = _batched_in(h_batched, "h_batched")
    dev = h_batched.device
    _need(expert_num_tokens, "expert_num_tokens", torch.int32, (E_l,), dev)
    if w2.E_l != E_l or w2.N != H or w2.K != I:
        raise ValueError(f"w2 must be [E_l={E_l}, H={H}, I={I}]")
    if y_batched is None:
        y_batched = torch.empty((E_l, M, H), dtype=torch.bfloat16, device=dev)
    _need(y_batched, "y_batched", torch.bfloat16, (E_l, M, H), dev)
    ws, ws_bytes, _keep = _gemm_workspace(E_l * M, H, False, split, dev, stream, workspace)
    _check(lib().moe_grouped_gemm2_batched(
        h_batched.data_ptr(), expert_num_tokens.data_ptr(), E_l, M, max_rows, I, H, w2.ref(),
        y_batched.data_ptr(), ws, ws_bytes, _stream(stream)), "moe_grouped_gemm2_batched")
    return y_batched


def moe_grouped_gemm_workspace_size(R_pad: int, N_out: int, gated: bool) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_grouped_gemm_workspace_size(R_pad, N_out, int(bool(gated)), ctypes.byref(n)),
           "moe_grouped_gemm_workspace_size")
    return int(n.value)


def _gemm_workspace(R_pad: int, N_out: int, gated: bool, split: bool, dev, stream,
                    workspace: Optional[torch.Tensor] = None):
    """(pointer, bytes, tensor) of the split-reduction workspace: the caller's,
    a fresh one, or (None, 0, None)."""
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, device=dev)
        return workspace.data_ptr(), workspace.numel(), workspace
    n = moe_grouped_gemm_workspace_size(R_pad, N_out, gated) if split else 0
    if n == 0:
        return None, 0, None
    buf = torch.empty(n, dtype=torch.uint8, device=dev)
    _hold(buf, stream)
    return buf.data_ptr(), n, buf


def moe_grouped_gemm1_act(a_perm: torch.Tensor, offsets: torch.Tensor, w1: Weights, I: int,
                          h: Optional[torch.Tensor] = None, activation=ACT_SILU,
                          stream=None, split: bool = True,
                          workspace: Optional[torch.Tensor] = None,
                          activation_clamp: Optional[float] = None) -> torch.Tensor:
    """h[r] = act(a_perm[r] W1g[e]^T) * (a_perm[r] W1u[e]^T) -> bf16 [R_pad, I]
    (act "silu" or "gelu"; activation_clamp > 0 clamps gate and up first).

    workspace: uint8 scratch (moe_grouped_gemm_workspace_size bytes) that lets
    few-row calls split the reduction; without one, split=True allocates it."""
    _need(a_perm, "a_perm", torch.bfloat16)
    R_pad, H = a_perm.shape
    dev = a_perm.device
    _need(offsets, "offsets", torch.int32, (w1.E_l + 1,), dev)
    if w1.N != 2 * I or w1.K != H:
        raise ValueError(f"w1 must be [E_l, 2I={2 * I}, H={H}]")
    if h is None:
        h = torch.empty((R_pad, I), dtype=torch.bfloat16, device=dev)
    _need(h, "h", torch.bfloat16, (R_pad, I), dev)
    ws, ws_bytes, _keep = _gemm_workspace(R_pad, I, True, split, dev, stream, workspace)
    _check(lib().moe_grouped_gemm1_act(a_perm.data_ptr(), offsets.data_ptr(), w1.E_l, R_pad, H, I,
                                       w1.ref(), _act(activation),
                                       0.0 if activation_clamp is None else float(activation_clamp),
                                       h.data_ptr(), ws, ws_bytes, _stream(stream)),
           "moe_grouped_gemm1_act")
    return h



def moe_grouped_gemm1_act_gathered(x: torch.Tensor, inv: torch.Tensor, k: int,
                                   offsets: torch.Tensor, w1: Weights, I: int,
                                   h: Optional[torch.Tensor] = None, activation=ACT_SILU,
                                   stream=None, split: bool = True,
                                   workspace: Optional[torch.Tensor] = None,
                                   activation_clamp: Optional[float] = None) -> torch.Tensor:
    """moe_grouped_gemm1_act on rows read straight from the tokens: permuted row
    r is x[inv[r] // k] (inv from moe_permute) -> bf16 [R_pad, I], R_pad = inv's length."""
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be [T, H]")
    T, H = x.shape
    dev = x.device
    _need(inv, "inv", torch.int32, device=dev)
    R_pad = inv.numel()
    _need(offsets, "offsets", torch.int32, (w1.E_l + 1,), dev)
    if w1.N != 2 * I or w1.K != H:
        raise ValueError(f"w1 must be [E_l, 2I={2 * I}, H={H}]")
    if h is None:
        h = torch.empty((R_pad, I), dtype=torch.bfloat16, device=dev)
    _need(h, "h", torch.bfloat16, (R_pad, I), dev)
    ws, ws_bytes, _keep = _gemm_workspace(R_pad, I, True, split, dev, stream, workspace)
    _check(lib().moe_grouped_gemm1_act_gathered(
        x.data_ptr(), inv.data_ptr(), T, k, offsets.data_ptr(), w1.E_l, R_pad, H, I, w1.ref(),
        _act(activation), 0.0 if activation_clamp is None else float(activation_clamp),
        h.data_ptr(), ws, ws_bytes, _stream(stream)), "moe_grouped_gemm1_act_gathered")
    return h

def moe_route_permute_gemm1_act(logits: torch.Tensor, x: torch.Tensor, k: int, w1: Weights,
                                I: int, score_fn: int = SOFTMAX, renormalize: bool = True,
                                rsf: float = 1.0, expert_map: Optional[torch.Tensor] = None,
                                R_pad: Optional[int] = None,
                                topk_ids: Optional[torch.Tensor] = None,
                                topk_weights: Optional[torch.Tensor] = None,
                                map: Optional[torch.Tensor] = None,
                                offsets: Optional[torch.Tensor] = None,
                                inv: Optional[torch.Tensor] = None,
                                h: Optional[torch.Tensor] = None, activation=ACT_SILU,
                                activation_clamp: Optional[float] = None, stream=None,
                                split: bool = True, workspace: Optional[torch.Tensor] = None):
    """Router, permute map and GEMM1 on the token rows in one call (one kernel
    for small bf16 decode batches).  -> dict(topk_ids, topk_weights, map,
    offsets, inv, h, R_pad)."""
    _need(logits, "logits", torch.float32)
    _need(x, "x", torch.bfloat16)
    if logits.dim() != 2 or x.dim() != 2 or x.shape[0] != logits.shape[0]:
        raise ValueError("logits must be [T, E] and x [T, H]")
    T, E = logits.shape
    H = x.shape[1]
    dev = x.device
    E_l = w1.E_l
    if expert_map is not None:
        _need(expert_map, "expert_map", torch.int32, (E,), dev)
    if w1.N != 2 * I or w1.K != H:
        raise ValueError(f"w1 must be [E_l, 2I={2 * I}, H={H}]")
    R_pad = moe_permuted_rows(T, k) if R_pad is None else R_pad
    out = {}
    for name, t, dt, shape in [("topk_ids", topk_ids, torch.int32, (T, k)),
                               ("topk_weights", topk_weights, torch.float32, (T, k)),
                               ("map", map, torch.int32, (T, k)),
                               ("offsets", offsets, torch.int32, (E_l + 1,)),
                               ("inv", inv, torch.int32, (R_pad,)),
                               ("h", h, torch.bfloat16, (R_pad, I))]:
        if t is None:
            t = torch.empty(shape, dtype=dt, device=dev)
        _need(t, name, dt, shape, dev)
        out[name] = t
    ws, ws_bytes, _keep = _gemm_workspace(R_pad, I, True, split, dev, stream, workspace)
    _check(lib().moe_route_permute_gemm1_act(
        logits.data_ptr(), x.data_ptr(), T, H, I, E, E_l, k, score_fn, int(bool(renormalize)),
        float(rsf), _ptr(expert_map), R_pad, w1.ref(), _act(activation),
        0.0 if activation_clamp is None else float(activation_clamp),
        out["topk_ids"].data_ptr(), out["topk_weights"].data_ptr(), out["map"].data_ptr(),
        out["offsets"].data_ptr(), out["inv"].data_ptr(), out["h"].data_ptr(), ws, ws_bytes,
        _stream(stream)), "moe_route_permute_gemm1_act")
    out["R_pad"] = R_pad
    return out


def moe_grouped_gemm2(h: torch.Tensor, offsets: torch.Tensor, w2: Weights, H: int,
                      y: Optional[torch.Tensor] = None, stream=None,
                      split: bool = True, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[r] = h[r] W2[e]^T -> bf16 [R_pad, H] (unweighted gemm2_permuted)."""
    _need(h, "h", torch.bfloat16)
    R_pad, I = h.shape
    dev = h.device
    _need(offsets, "offsets", torch.int32, (w2.E_l + 1,), dev)
    if w2.N != H or w2.K != I:
        raise ValueError(f"w2 must be [E_l, H={H}, I={I}]")
    if y is None:
        y = torch.empty((R_pad, H), dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, (R_pad, H), dev)
    ws, ws_bytes, _keep = _gemm_workspace(R_pad, H, False, split, dev, stream, workspace)
    _check(lib().moe_grouped_gemm2(h.data_ptr(), offsets.data_ptr(), w2.E_l, R_pad, I, H, w2.ref(),
                                   y.data_ptr(), ws, ws_bytes, _stream(stream)), "moe_grouped_gemm2")
    return y


def moe_finalize(gemm2_permuted: torch.Tensor, expert_weights: Optional[torch.Tensor],
                 map: torch.Tensor, rsf_fin: float = 1.0, shared: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out[t] = rsf_fin * sum_{map>=0} w * Y[map] + shared[t] -> bf16 [T, H]
    (expert_weights None: every weight 1, as after apply_router_weight_on_input).
    gemm2_permuted may be [R, H] or batched [E_l, max_tokens, H]."""
    _need(gemm2_permuted, "gemm2_permuted", torch.bfloat16)
    if gemm2_permuted.dim() == 3:
        gemm2_permuted = gemm2_permuted.view(-1, gemm2_permuted.shape[2])
    if gemm2_permuted.dim() != 2:
        raise ValueError("gemm2_permuted must be rank-2")
    H = gemm2_permuted.shape[1]
    dev = gemm2_permuted.device
    _need(map, "map", torch.int32, device=dev)
    if map.dim() != 2:
        raise ValueError("map must be [T, k]")
    T, k = map.shape
    w_ptr, wdt = _weights_arg(expert_weights, T, k, dev)
    if shared is not None:
        _need(shared, "shared", torch.bfloat16, (T, H), dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (T, H), dev)
    _check(lib().moe_finalize(gemm2_permuted.data_ptr(), gemm2_permuted.shape[0], w_ptr, wdt,
                              map.data_ptr(), T, k, H, float(rsf_fin), _ptr(shared),
                              out.data_ptr(), _stream(stream)), "moe_finalize")
    return out


def moe_finalize_add_rmsnorm(gemm2_permuted: torch.Tensor, expert_weights: Optional[torch.Tensor],
                             map: torch.Tensor, residual: torch.Tensor, gamma: torch.Tensor,
                             eps: float = 1e-6, rsf_fin: float = 1.0,
                             shared: Optional[torch.Tensor] = None,
                             out: Optional[torch.Tensor] = None, stream=None):
    """Fused tail: residual += finalize(...) (in place); out = RMSNorm(residual) * gamma.
    -> (out bf16 [T, H], residual).  gemm2_permuted as for moe_finalize."""
    _need(gemm2_permuted, "gemm2_permuted", torch.bfloat16)
    if gemm2_permuted.dim() == 3:
        gemm2_permuted = gemm2_permuted.view(-1, gemm2_permuted.shape[2])
    if gemm2_permuted.dim() != 2:
        raise ValueError("gemm2_permuted must be rank-2")
    H = gemm2_permuted.shape[1]
    dev = gemm2_permuted.device
    _need(map, "map", torch.int32, device=dev)
    if map.dim() != 2:
        raise ValueError("map must be [T, k]")
    T, k = map.shape
    w_ptr, wdt = _weights_arg(expert_weights, T, k, dev)
    _need(residual, "residual", torch.bfloat16, (T, H), dev)
    _need(gamma, "gamma", torch.bfloat16, (H,), dev)
    if shared is not None:
        _need(shared, "shared", torch.bfloat16, (T, H), dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (T, H), dev)
    _check(lib().moe_finalize_add_rmsnorm(gemm2_permuted.data_ptr(), gemm2_permuted.shape[0],
                                          w_ptr, wdt,
                                          map.data_ptr(), T, k, H, float(rsf_fin), _ptr(shared),
                                          residual.data_ptr(), gamma.data_ptr(), float(eps),
                                          out.data_ptr(), _stream(stream)),
           "moe_finalize_add_rmsnorm")
    return out, residual


def _workspace(nbytes: int, dev, workspace: Optional[torch.Tensor], stream=None) -> torch.Tensor:
    if workspace is None:
        workspace = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=dev)
        _hold(workspace, stream)
    _need(workspace, "workspace", torch.uint8, device=dev)
    if workspace.numel() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return workspace


def moe_fused_experts_unfinalized(logits: torch.Tensor, x: torch.Tensor, w1: Weights, w2: Weights,
                                  k: int, score_fn: int = SOFTMAX, renormalize: bool = True,
                                  rsf: float = 1.0, expert_map: Optional[torch.Tensor] = None,
                                  R_pad: Optional[int] = None,
                                  workspace: Optional[torch.Tensor] = None,
                                  gemm2_permuted: Optional[torch.Tensor] = None,
                                  expert_weights: Optional[torch.Tensor] = None,
                                  map: Optional[torch.Tensor] = None, stream=None,
                                  activation=ACT_SILU, activation_clamp: Optional[float] = None,
                                  apply_router_weight_on_input: bool = False,
                                  batched_max_tokens: int = 0, fp8=False,
                                  a1_scale: Optional[torch.Tensor] = None,
                                  a2_scale: Optional[torch.Tensor] = None):
    """-> (gemm2_permuted bf16 [R_pad, H], expert_weights bf16 [T, k], map int32 [T, k]).
    batched_max_tokens > 0: batched experts format, R_pad = E_l * batched_max_tokens."""
    _need(logits, "logits", torch.float32)
    _need(x, "x", torch.bfloat16, device=logits.device)
    T, E = logits.shape
    H = x.shape[1]
    I = w2.K
    dev = x.device
    if R_pad is None:
        R_pad = w1.E_l * batched_max_tokens if batched_max_tokens else moe_permuted_rows(T, k)
    if gemm2_permuted is None:
        gemm2_permuted = torch.empty((R_pad, H), dtype=torch.bfloat16, device=dev)
    if expert_weights is None:
        expert_weights = torch.empty((T, k), dtype=torch.bfloat16, device=dev)
    if map is None:
        map = torch.empty((T, k), dtype=torch.int32, device=dev)
    _need(gemm2_permuted, "gemm2_permuted", torch.bfloat16, (R_pad, H), dev)
    _need(expert_weights, "expert_weights", torch.bfloat16, (T, k), dev)
    _need(map, "map", torch.int32, (T, k), dev)
    if expert_map is not None:
        _need(expert_map, "expert_map", torch.int32, (E,), dev)
    nbytes = (moe_workspace_size(T, k, E, w1.E_l, H, I, w1.dtype,
                                 batched_max_tokens=batched_max_tokens, fp8=fp8) if T > 0 else 0)
    ws = _workspace(nbytes, dev, workspace, stream)
    _check(lib().moe_fused_experts_unfinalized(
        logits.data_ptr(), x.data_ptr(), T, H, I, E, w1.E_l, k, score_fn, int(bool(renormalize)),
        float(rsf), _ptr(expert_map), w1.ref(), w2.ref(),
        _options(activation, activation_clamp, apply_router_weight_on_input, 0,
                 batched_max_tokens, fp8, a1_scale, a2_scale), R_pad,
        gemm2_permuted.data_ptr(),
        expert_weights.data_ptr(), map.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream)),
        "moe_fused_experts_unfinalized")
    return gemm2_permuted, expert_weights, map


def moe_fused_experts_unfinalized_noalloc(logits: torch.Tensor, x: torch.Tensor, w1: Weights,
                                          w2: Weights, k: int, score_fn: int = SOFTMAX,
                                          renormalize: bool = True, rsf: float = 1.0,
                                          expert_map: Optional[torch.Tensor] = None,
                                          R_pad: Optional[int] = None,
                                          gemm2_permuted: Optional[torch.Tensor] = None,
                                          expert_weights: Optional[torch.Tensor] = None,
                                          map: Optional[torch.Tensor] = None, stream=None,
                                          activation=ACT_SILU,
                                          activation_clamp: Optional[float] = None,
                                          apply_router_weight_on_input: bool = False,
                                          batched_max_tokens: int = 0, fp8=False,
                                          a1_scale: Optional[torch.Tensor] = None,
                                          a2_scale: Optional[torch.Tensor] = None):
    """moe_fused_experts_unfinalized on the library's static device scratch (no
    workspace): the library allocates nothing.  Outputs the caller does not
    pass are allocated here by torch; pass all three to allocate nothing at
    all.  -> (gemm2_permuted, expert_weights, map)."""
    _need(logits, "logits", torch.float32)
    _need(x, "x", torch.bfloat16, device=logits.device)
    T, E = logits.shape
    H = x.shape[1]
    I = w2.K
    dev = x.device
    if R_pad is None:
        R_pad = w1.E_l * batched_max_tokens if batched_max_tokens else moe_permuted_rows(T, k)
    if gemm2_permuted is None:
        gemm2_permuted = torch.empty((R_pad, H), dtype=torch.bfloat16, device=dev)
    if expert_weights is None:
        expert_weights = torch.empty((T, k), dtype=torch.bfloat16, device=dev)
    if map is None:
        map = torch.empty((T, k), dtype=torch.int32, device=dev)
    _need(gemm2_permuted, "gemm2_permuted", torch.bfloat16, (R_pad, H), dev)
    _need(expert_weights, "expert_weights", torch.bfloat16, (T, k), dev)
    _need(map, "map", torch.int32, (T, k), dev)
    if expert_map is not None:
        _need(expert_map, "expert_map", torch.int32, (E,), dev)
    _check(lib().moe_fused_experts_unfinalized_noalloc(
        logits.data_ptr(), x.data_ptr(), T, H, I, E, w1.E_l, k, score_fn, int(bool(renormalize)),
        float(rsf), _ptr(expert_map), w1.ref(), w2.ref(),
        _options(activation, activation_clamp, apply_router_weight_on_input, 0,
                 batched_max_tokens, fp8, a1_scale, a2_scale), R_pad,
        gemm2_permuted.data_ptr(), expert_weights.data_ptr(), map.data_ptr(), _stream(stream)),
        "moe_fused_experts_unfinalized_noalloc")
    return gemm2_permuted, expert_weights, map


def moe_fused_experts(logits: torch.Tensor, x: torch.Tensor, w1: Weights, w2: Weights, k: int,
                      score_fn: int = SOFTMAX, renormalize: bool = True, rsf: float = 1.0,
                      expert_map: Optional[torch.Tensor] = None,
                      ws1: Optional[torch.Tensor] = None, ws2: Optional[torch.Tensor] = None,
                      rsf_fin: float = 1.0, out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None,
                      activation=ACT_SILU, activation_clamp: Optional[float] = None,
                      apply_router_weight_on_input: bool = False, chunk_tokens: int = 0,
                      inplace: bool = False, batched_max_tokens: int = 0, fp8=False,
                      a1_scale: Optional[torch.Tensor] = None,
                      a2_scale: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The whole layer, finalized (optionally with a shared expert ws1 [2Is, H], ws2 [H, Is]).

    chunk_tokens > 0 runs it over chunks of that many tokens with a workspace
    sized for one chunk; inplace writes the output over x."""
    _need(logits, "logits", torch.float32)
    _need(x, "x", torch.bfloat16, device=logits.device)
    T, E = logits.shape
    H = x.shape[1]
    I = w2.K
    dev = x.device
    shared_I = 0
    if ws1 is not None or ws2 is not None:
        _need(ws1, "ws1", torch.bfloat16, device=dev)
        _need(ws2, "ws2", torch.bfloat16, device=dev)
        shared_I = ws2.shape[1]
        if tuple(ws1.shape) != (2 * shared_I, H) or tuple(ws2.shape) != (H, shared_I):
            raise ValueError("shared weights must be ws1 [2*Is, H] and ws2 [H, Is]")
    if expert_map is not None:
        _need(expert_map, "expert_map", torch.int32, (E,), dev)
    if inplace:
        out = x
    elif out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (T, H), dev)
    nbytes = 0
    if T > 0:
        nbytes = moe_workspace_size(T, k, E, w1.E_l, H, I, w1.dtype, shared_I, chunk_tokens,
                                    batched_max_tokens, fp8)
    ws = _workspace(nbytes, dev, workspace, stream)
    _check(lib().moe_fused_experts(
        logits.data_ptr(), x.data_ptr(), T, H, I, E, w1.E_l, k, score_fn, int(bool(renormalize)),
        float(rsf), _ptr(expert_map), w1.ref(), w2.ref(), shared_I, _ptr(ws1), _ptr(ws2),
        float(rsf_fin),
        _options(activation, activation_clamp, apply_router_weight_on_input, chunk_tokens,
                 batched_max_tokens, fp8, a1_scale, a2_scale),
        out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream)),
        "moe_fused_experts")
    return out
