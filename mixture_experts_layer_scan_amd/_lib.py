"""Loader of the HIP library ``libmoe_mi355x.so`` (ctypes prototypes).

The library is required: there is no fallback.  A missing or unloadable
library raises at first use with the command that builds it.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_mi355x.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe.h")


class MoeWeightsC(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("data", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class MoeLayerOptionsC(ctypes.Structure):
    _fields_ = [("activation", ctypes.c_int32), ("activation_clamp", ctypes.c_float),
                ("apply_router_weight_on_input", ctypes.c_int32),
                ("chunk_tokens", ctypes.c_int32), ("batched_max_tokens", ctypes.c_int32),
                ("act_quant", ctypes.c_int32), ("a1_scale", ctypes.c_void_p),
                ("a2_scale", ctypes.c_void_p)]


_i32, _i64, _f32, _vp, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
_Wp = ctypes.POINTER(MoeWeightsC)
_Op = ctypes.POINTER(MoeLayerOptionsC)

PROTOTYPES = {
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_permuted_rows": (_i64, [_i64, _i32]),
    "moe_workspace_size": (ctypes.c_int, [_i64, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _Op,
                                          ctypes.POINTER(_sz)]),
    "moe_shared_workspace_size": (ctypes.c_int, [_i64, _i32, _i32, ctypes.POINTER(_sz)]),
    "moe_route_topk": (ctypes.c_int, [_vp, _i64, _i32, _i32, _i32, _i32, _f32, _vp, _vp, _vp]),
    "moe_route_permute": (ctypes.c_int, [_vp, _i64, _i32, _i32, _i32, _i32, _f32, _vp, _i32, _i64,
                                         _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_route_permute_gemm1_act": (ctypes.c_int, [_vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32,
                                                   _i32, _i32, _f32, _vp, _i64, _vp, _i32, _f32,
                                                   _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_permute": (ctypes.c_int, [_vp, _vp, _i64, _i32, _i32, _i32, _vp, _i32, _i64, _vp, _vp,
                                   _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_grouped_gemm1_act": (ctypes.c_int, [_vp, _vp, _i32, _i64, _i32, _i32, _Wp, _i32, _f32,
                                             _vp, _vp, _sz, _vp]),
    "moe_quantize_fp8": (ctypes.c_int, [_vp, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_permute_fp8": (ctypes.c_int, [_vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _i32, _i64,
                                       _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_grouped_gemm1_act_fp8": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i64, _i32, _i32, _Wp, _i32,
                                                 _f32, _vp, _vp, _sz, _vp]),
    "moe_grouped_gemm2_fp8": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i64, _i32, _i32, _Wp, _vp, _vp,
                                             _sz, _vp]),
    "moe_quantize_fp8_blockwise": (ctypes.c_int, [_vp, _i64, _i32, _vp, _vp, _vp, _i64, _vp]),
    "moe_permute_fp8_blockwise": (ctypes.c_int, [_vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _i32,
                                                 _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_grouped_gemm1_act_fp8_blockwise": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i64, _i32, _i32,
                                                           _Wp, _i32, _f32, _vp, _vp, _sz, _vp]),
    "moe_grouped_gemm2_fp8_blockwise": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i64, _i32, _i32, _Wp,
                                                       _vp, _vp, _sz, _vp]),
    "moe_grouped_gemm1_act_fp8_gathered": (ctypes.c_int, [_vp, _vp, _i32, _vp, _i64, _i32, _vp,
                                                          _i32, _i64, _i32, _i32, _Wp, _i32, _f32,
                                                          _vp, _vp, _sz, _vp]),
    "moe_quantize_fp8x2": (ctypes.c_int, [_vp, _i64, _i32, _vp, _vp, _vp, _vp, _vp]),
    "moe_grouped_gemm1_act_fp8x2": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i64, _i32, _i32, _Wp,
                                                   _i32, _f32, _vp, _vp, _sz, _vp]),
    "moe_grouped_gemm2_fp8x2": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i64, _i32, _i32, _Wp, _vp,
                                               _vp, _sz, _vp]),
    "moe_permute_batched": (ctypes.c_int, [_vp, _vp, _i64, _i32, _i32, _i32, _vp, _i32, _i32,
                                           _vp, _vp, _vp, _vp, _vp]),
    "moe_grouped_gemm1_act_batched": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i64, _i32, _i32, _Wp,
                                                     _i32, _f32, _vp, _vp, _sz, _vp]),
    "moe_grouped_gemm2_batched": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i64, _i32, _i32, _Wp,
                                                 _vp, _vp, _sz, _vp]),
    "moe_grouped_gemm2": (ctypes.c_int, [_vp, _vp, _i32, _i64, _i32, _i32, _Wp, _vp, _vp, _sz,
                                         _vp]),
    "moe_grouped_gemm1_act_gathered": (ctypes.c_int, [_vp, _vp, _i64, _i32, _vp, _i32, _i64, _i32,
                                                      _i32, _Wp, _i32, _f32, _vp, _vp, _sz, _vp]),
    "moe_finalize_add_rmsnorm": (ctypes.c_int, [_vp, _i64, _vp, _i32, _vp, _i64, _i32, _i32, _f32, _vp,
                                                _vp, _vp, _f32, _vp, _vp]),
    "moe_grouped_gemm_workspace_size": (ctypes.c_int, [_i64, _i32, _i32, ctypes.POINTER(_sz)]),
    "moe_finalize": (ctypes.c_int, [_vp, _i64, _vp, _i32, _vp, _i64, _i32, _i32, _f32, _vp, _vp,
                                    _vp]),
    "moe_fused_experts_unfinalized": (ctypes.c_int, [_vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32,
                                                     _i32, _i32, _f32, _vp, _Wp, _Wp, _Op, _i64,
                                                     _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_fused_experts_unfinalized_noalloc": (ctypes.c_int, [_vp, _vp, _i64, _i32, _i32, _i32,
                                                             _i32, _i32, _i32, _i32, _f32, _vp,
                                                             _Wp, _Wp, _Op, _i64, _vp, _vp, _vp,
                                                             _vp]),
    "moe_fused_experts": (ctypes.c_int, [_vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                         _f32, _vp, _Wp, _Wp, _i32, _vp, _vp, _f32, _Op, _vp, _vp,
                                         _sz, _vp]),
}

_lib = None


def header_functions(path: str = HEADER):
    """Names of the functions include/moe.h declares."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m mixture_experts_layer_scan_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in PROTOTYPES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib
