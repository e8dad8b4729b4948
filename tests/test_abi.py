"""The C ABI without a GPU: the library loads, exports every function that
include/moe.h declares, and rejects bad arguments on the host before any HIP
call (so these run on a machine with no GPU).  The error cases follow the
checks of convert_flashinfer_moe_output in vLLM's MoE output contract."""
import ctypes

import pytest

from mixture_experts_layer_scan_amd import _lib

OK, INVALID, UNSUPPORTED, SIZE, MISALIGNED, DEVICE, CONFLICT, HIP = 0, -1, -2, -3, -4, -5, -6, -7

P = 0x10000  # a fake, 16-byte aligned "device" pointer: never dereferenced here


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_exports_every_declared_function(L):
    declared = _lib.header_functions()
    assert len(declared) >= 12
    for name in declared:
        assert hasattr(L, name), name
    assert set(_lib.PROTOTYPES) == set(declared)


def test_status_strings(L):
    for s in (OK, INVALID, UNSUPPORTED, SIZE, MISALIGNED, DEVICE, CONFLICT, HIP):
        assert L.moe_status_string(s)
    assert L.moe_status_string(-99) == b"unknown status"


def test_permuted_rows(L):
    assert L.moe_permuted_rows(0, 8) == 0
    assert L.moe_permuted_rows(1, 8) == 128
    assert L.moe_permuted_rows(16, 8) == 128
    assert L.moe_permuted_rows(17, 8) == 256
    assert L.moe_permuted_rows(4096, 2) == 8192


def _ws(L, T, k, E, El, H, I, dt=0, sI=0, opts=None):
    n = ctypes.c_size_t(0)
    s = L.moe_workspace_size(T, k, E, El, H, I, dt, sI, opts, ctypes.byref(n))
    return s, n.value


def test_workspace_size(L):
    s, n = _ws(L, 2048, 8, 256, 256, 7168, 2048)
    assert s == OK
    R = 2048 * 8
    assert n >= R * (7168 + 2048) * 2 + 3 * R * 4
    assert _ws(L, -1, 8, 256, 256, 7168, 2048)[0] == INVALID
    assert _ws(L, 16, 0, 8, 8, 128, 256)[0] == INVALID
    assert _ws(L, 16, 2, 8, 8, 100, 256)[0] == INVALID      # H not a multiple of 64
    assert _ws(L, 16, 2, 8, 9, 128, 256)[0] == INVALID      # E_l > E
    assert _ws(L, 16, 2, 8, 8, 128, 256, 7)[0] == UNSUPPORTED
    # the shared expert's part, chunking and the batched experts format
    s0, n0 = _ws(L, 2048, 8, 256, 256, 7168, 2048)
    s1, n1 = _ws(L, 2048, 8, 256, 256, 7168, 2048, sI=2048)
    ns = ctypes.c_size_t(0)
    assert L.moe_shared_workspace_size(2048, 7168, 2048, ctypes.byref(ns)) == OK
    assert s1 == OK and n1 == n0 + ns.value
    _, n512 = _ws(L, 512, 8, 256, 256, 7168, 2048)
    assert _ws(L, 2048, 8, 256, 256, 7168, 2048, opts=_opts(chunk=512)) == (OK, n512)
    assert _ws(L, 2048, 8, 256, 256, 7168, 2048, opts=_opts(chunk=4096)) == (OK, n0)
    s, nb = _ws(L, 64, 8, 256, 32, 7168, 2048, opts=_opts(batched=64))
    assert s == OK and nb >= 32 * 64 * (7168 + 2048) * 2
    assert _ws(L, 64, 8, 256, 32, 7168, 2048, opts=_opts(batched=-1))[0] == INVALID
    n = ctypes.c_size_t(0)
    assert L.moe_shared_workspace_size(2048, 7168, 0, ctypes.byref(n)) == OK and n.value == 0
    assert L.moe_shared_workspace_size(2048, 7168, 2048, ctypes.byref(n)) == OK
    assert n.value >= 2048 * (7168 + 2048) * 2


def test_route_errors(L):
    r = L.moe_route_topk
    assert r(P, -1, 8, 2, 0, 1, 1.0, P, P, None) == INVALID
    assert b"non-negative" in L.moe_last_error()
    assert r(P, 4, 8, 0, 0, 1, 1.0, P, P, None) == INVALID
    assert b"positive" in L.moe_last_error()
    assert r(P, 4, 8, 9, 0, 1, 1.0, P, P, None) == INVALID   # k > E
    assert r(P, 4, 2048, 2, 0, 1, 1.0, P, P, None) == INVALID  # E > 1024
    assert r(P, 4, 8, 2, 5, 1, 1.0, P, P, None) == UNSUPPORTED
    assert r(P + 4, 4, 8, 2, 0, 1, 1.0, P, P, None) == MISALIGNED
    assert r(None, 4, 8, 2, 0, 1, 1.0, P, P, None) == INVALID
    assert r(None, 0, 8, 2, 0, 1, 1.0, None, None, None) == OK  # T = 0: nothing to do


def test_route_permute_errors(L):
    f = L.moe_route_permute
    # (logits, T, E, k, score, renorm, rsf, emap, E_l, R_pad, ids, w, map, offsets, inv, stream)
    assert f(P, -1, 8, 2, 0, 1, 1.0, None, 8, 0, P, P, P, P, None, None) == INVALID
    assert f(P, 4, 8, 9, 0, 1, 1.0, None, 8, 36, P, P, P, P, None, None) == INVALID  # k > E
    assert f(P, 4, 8, 2, 5, 1, 1.0, None, 8, 8, P, P, P, P, None, None) == UNSUPPORTED
    assert f(P, 4, 8, 2, 0, 1, 1.0, None, 4, 8, P, P, P, P, None, None) == INVALID  # E_l != E, no map
    assert f(P, 4, 8, 2, 0, 1, 1.0, None, 8, 7, P, P, P, P, None, None) == SIZE     # R_pad < T * k
    assert f(P, 4, 8, 2, 0, 1, 1.0, None, 8, 8, P, P, P, None, None, None) == INVALID  # no offsets
    assert f(None, 4, 8, 2, 0, 1, 1.0, None, 8, 8, P, P, P, P, None, None) == INVALID
    assert f(P, 4, 8, 2, 0, 1, 1.0, None, 8, 8, P + 4, P, P, P, None, None) == MISALIGNED


def test_route_permute_gemm1_errors(L):
    f = L.moe_route_permute_gemm1_act
    # (logits, x, T, H, I, E, E_l, k, score, renorm, rsf, emap, R_pad, w1, act, clamp,
    #  ids, w, map, offsets, inv, h, workspace, workspace_bytes, stream)
    w = _w()
    ok = dict(T=4, H=128, I=256, E=8, E_l=8, k=2, R_pad=128)

    def call(**kw):
        a = dict(ok, **kw)
        return f(P, P * 2, a["T"], a["H"], a["I"], a["E"], a["E_l"], a["k"], kw.get("score", 0), 1,
                 1.0, None, a["R_pad"], kw.get("w1", w), kw.get("act", 0), kw.get("clamp", 0.0),
                 P * 3, P * 4, P * 5, kw.get("offsets", P * 6), kw.get("inv", P * 7),
                 kw.get("h", P * 64), None, 0, None)
    assert call(T=-1) == INVALID
    assert call(k=9) == INVALID                  # k > E
    assert call(score=5) == UNSUPPORTED
    assert call(E_l=4) == INVALID                # no expert map, E_l != E
    assert call(R_pad=7) == SIZE                 # R_pad < T * k
    assert call(H=100) == INVALID                # H not a multiple of 64
    assert call(act=3) == UNSUPPORTED
    assert call(offsets=None) == INVALID
    assert call(inv=None) == INVALID
    assert call(h=P * 7) == CONFLICT             # h over the inverse map
    assert call(w1=None) == INVALID


def test_permute_errors(L):
    f = L.moe_permute
    # R_pad < T * k
    assert f(P, None, 16, 2, 8, 8, P, 128, 31, P, P, P, P, None, None, 0, None) == SIZE
    # no expert map but E_l != E
    assert f(P, None, 16, 2, 8, 4, P, 128, 32, P, P, P, P, None, None, 0, None) == INVALID
    # H not a multiple of 8 with a gather
    assert f(P, None, 16, 2, 8, 8, P, 100, 32, P, P, P, P, None, None, 0, None) == INVALID
    # x_perm overlapping x
    assert f(P, None, 16, 2, 8, 8, P, 128, 32, P, P, P, P + 64, None, None, 0, None) == CONFLICT


def _w(dtype=0, data=P, scales=None):
    return ctypes.byref(_lib.MoeWeightsC(dtype, data, scales))


def test_gemm_errors(L):
    g1 = L.moe_grouped_gemm1_act
    assert g1(P, P, 8, 128, 100, 256, _w(), 0, 0.0, P * 64, None, 0, None) == INVALID  # H % 64
    assert g1(P, P, 8, 128, 128, 256, _w(), 3, 0.0, P * 64, None, 0, None) == UNSUPPORTED
    assert g1(P, P, 8, 128, 128, 256, _w(9), 0, 0.0, P * 64, None, 0, None) == UNSUPPORTED
    assert g1(P, P, 8, 128, 128, 256, None, 0, 0.0, P * 64, None, 0, None) == INVALID
    assert g1(P, P, 8, 128, 128, 256, _w(2, P, None), 0, 0.0, P * 64, None, 0, None) == INVALID  # MXFP4, no scales
    assert g1(P, P, 8, 128, 128, 256, _w(0, P, P), 0, 0.0, P * 64, None, 0, None) == INVALID  # bf16 with scales
    assert g1(P, P, 8, 128, 128, 256, _w(), 0, 0.0, P, None, 0, None) == CONFLICT  # h == a_perm
    assert g1(P, P, 0, 128, 128, 256, _w(), 0, 0.0, P * 64, None, 0, None) == INVALID  # E_l = 0
    assert g1(P, P, 8, 128, 128, 256, _w(), 1, -0.5, P * 64, None, 0, None) == INVALID  # clamp < 0
    assert g1(P, P, 8, 128, 128, 256, _w(), 2, 0.0, P * 64, None, 0, None) == UNSUPPORTED
    g2 = L.moe_grouped_gemm2
    assert g2(P, P, 8, 128, 256, 130, _w(), P * 64, None, 0, None) == INVALID
    # one expert's weights over 4 GiB cannot be addressed
    assert g2(P, P, 8, 128, 65536, 65536, _w(), P * 64, None, 0, None) == INVALID


def test_finalize_errors(L):
    f = L.moe_finalize
    assert f(P, 32, P, 1, P, -1, 2, 128, 1.0, None, P * 8, None) == INVALID
    assert f(P, 32, P, 1, P, 16, 0, 128, 1.0, None, P * 8, None) == INVALID
    assert f(P, 32, P, 3, P, 16, 2, 128, 1.0, None, P * 8, None) == UNSUPPORTED  # int32 weights
    assert f(P, 32, P, 1, P, 16, 2, 130, 1.0, None, P * 8, None) == INVALID
    assert f(P, 32, P, 1, P, 16, 2, 128, 1.0, None, P + 256, None) == CONFLICT  # out inside y
    # the check spans y_rows rows of y (here 33 x 256 bytes), not T * k
    assert f(P, 33, P, 1, P, 16, 2, 128, 1.0, None, P + 32 * 256, None) == CONFLICT
    assert f(P, -1, P, 1, P, 16, 2, 128, 1.0, None, P * 8, None) == INVALID  # y_rows < 0
    assert f(P, 1 << 60, P, 1, P, 16, 2, 128, 1.0, None, P * 8, None) == INVALID  # y too large
    assert f(P, 32, P, 1, P, 16, 2, 128, 1.0, P * 4 + 16, P * 4, None) == CONFLICT  # partial alias
    assert f(P, 32, P, 1, P, 0, 2, 128, 1.0, None, None, None) == OK  # T = 0


def test_finalize_add_rmsnorm_errors(L):
    f = L.moe_finalize_add_rmsnorm
    # (y, y_rows, w, wdt, map, T, k, H, rsf, shared, residual, gamma, eps, out, stream)
    R, G, O = P * 8, P * 16, P * 24
    assert f(P, 32, P, 1, P, -1, 2, 128, 1.0, None, R, G, 1e-6, O, None) == INVALID
    assert f(P, 32, P, 1, P, 16, 0, 128, 1.0, None, R, G, 1e-6, O, None) == INVALID
    assert f(P, 32, P, 1, P, 16, 2, 130, 1.0, None, R, G, 1e-6, O, None) == INVALID
    assert f(P, 32, P, 1, P, 16, 2, 16392, 1.0, None, R, G, 1e-6, O, None) == INVALID  # H too large
    assert f(P, 32, P, 1, P, 16, 2, 128, 1.0, None, R, G, -1.0, O, None) == INVALID  # eps < 0
    assert f(P, 32, P, 3, P, 16, 2, 128, 1.0, None, R, G, 1e-6, O, None) == UNSUPPORTED
    assert f(P, 32, P, 1, P, 16, 2, 128, 1.0, None, None, G, 1e-6, O, None) == INVALID  # no residual
    assert f(P, 32, P, 1, P, 16, 2, 128, 1.0, None, R, None, 1e-6, O, None) == INVALID  # no gamma
    assert f(P, 32, P, 1, P, 16, 2, 128, 1.0, None, R, G, 1e-6, R, None) == CONFLICT  # out == residual
    assert f(P, 32, P, 1, P, 16, 2, 128, 1.0, R, R, G, 1e-6, O, None) == CONFLICT  # shared == residual
    assert f(P, 32, P, 1, P, 16, 2, 128, 1.0, None, R, G, 1e-6, P + 256, None) == CONFLICT  # out in y
    assert f(P, -1, P, 1, P, 16, 2, 128, 1.0, None, R, G, 1e-6, O, None) == INVALID  # y_rows < 0
    assert f(P, 32, P, 1, P, 0, 2, 128, 1.0, None, None, None, 1e-6, None, None) == OK  # T = 0


def test_fused_errors(L):
    u = L.moe_fused_experts_unfinalized
    args = dict(logits=P, x=P, T=16, H=128, I=256, E=8, El=8, k=2, score=0, renorm=1, rsf=1.0,
                emap=None, w1=_w(), w2=_w(), opts=None, R_pad=32, y=P, w=P, m=P, ws=P,
                wsb=1 << 30, s=None)

    def call(**kw):
        a = dict(args, **kw)
        return u(*a.values())
    assert call(T=-1) == INVALID
    assert call(k=0) == INVALID
    assert call(R_pad=31) == SIZE
    assert call(wsb=1024) == SIZE
    assert call(ws=P + 16) == MISALIGNED
    assert call(w1=_w(7, P, P)) == UNSUPPORTED
    assert call(El=4) == INVALID  # no map, E_l != E
    assert call(T=0) == OK
    assert call(opts=_opts(activation=2)) == UNSUPPORTED
    assert call(opts=_opts(clamp=-1.0)) == INVALID
    assert call(opts=_opts(clamp=float("nan"))) == INVALID
    assert call(opts=_opts(clamp=float("inf"))) == INVALID
    assert call(opts=_opts(weight_on_input=1)) == INVALID  # needs top_k = 1
    assert b"top_k = 1" in L.moe_last_error()
    assert call(opts=_opts(chunk=-4)) == INVALID
    assert call(opts=_opts(chunk=8)) == INVALID  # the deferred form takes no chunking


def _opts(activation=0, clamp=0.0, weight_on_input=0, chunk=0, batched=0, quant=0, a1=None,
          a2=None):
    return ctypes.byref(_lib.MoeLayerOptionsC(activation, clamp, weight_on_input, chunk, batched,
                                              quant, a1, a2))


def test_fused_finalized_errors(L):
    f = L.moe_fused_experts
    X, OUT = P * 1024, P * 2048
    args = dict(logits=P, x=X, T=16, H=128, I=256, E=8, El=8, k=2, score=0, renorm=1, rsf=1.0,
                emap=None, w1=_w(), w2=_w(), sI=0, ws1=None, ws2=None, rsf_fin=1.0, opts=None,
                out=OUT, ws=P * 4096, wsb=1 << 30, s=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(*a.values())
    assert call(out=X + 256) == CONFLICT          # partly over x
    assert b"x itself" in L.moe_last_error()
    assert call(ws=X) == CONFLICT                 # workspace over x
    assert call(opts=_opts(weight_on_input=1)) == INVALID
    assert call(k=1, opts=_opts(weight_on_input=1), wsb=16) == SIZE
    # chunking sizes the workspace for one chunk: 16 tokens in chunks of 4
    n4 = ctypes.c_size_t(0)
    assert L.moe_workspace_size(4, 2, 8, 8, 128, 256, 0, 0, None, ctypes.byref(n4)) == OK
    assert call(opts=_opts(chunk=4), wsb=n4.value - 256) == SIZE
    assert call(T=0, opts=_opts(chunk=4)) == OK


def test_batched_errors(L):
    pb = L.moe_permute_batched
    # (ids, emap, T, k, E, E_l, x, H, max_tokens, map, counts, x_batched, x_weights, stream)
    assert pb(P, None, 16, 2, 8, 8, P, 128, 0, P, P, P * 64, None, None) == INVALID  # capacity 0
    assert pb(P, None, 16, 2, 8, 8, P, 128, 1 << 28, P, P, P * 64, None, None) == INVALID
    assert pb(P, None, 16, 2, 8, 4, P, 128, 16, P, P, P * 64, None, None) == INVALID  # no map
    assert pb(P, None, 16, 2, 8, 8, P, 100, 16, P, P, P * 64, None, None) == INVALID  # H % 8
    assert pb(P, None, 16, 2, 8, 8, P, 128, 16, P, None, P * 64, None, None) == INVALID
    assert pb(P, None, 16, 2, 8, 8, P, 128, 16, P, P, P + 64, None, None) == CONFLICT
    g1 = L.moe_grouped_gemm1_act_batched
    # (a, counts, E_l, M, max_rows, H, I, w1, act, clamp, h, ws, wsb, stream)
    assert g1(P, P, 8, 0, 0, 128, 256, _w(), 0, 0.0, P * 64, None, 0, None) == INVALID
    assert g1(P, P, 8, 16, -1, 128, 256, _w(), 0, 0.0, P * 64, None, 0, None) == INVALID
    assert g1(P, P, 8, 16, 0, 128, 256, _w(), 5, 0.0, P * 64, None, 0, None) == UNSUPPORTED
    assert g1(P, P, 8, 16, 0, 128, 256, _w(), 0, 0.0, P, None, 0, None) == CONFLICT
    g2 = L.moe_grouped_gemm2_batched
    assert g2(P, P, 8, 16, 0, 256, 130, _w(), P * 64, None, 0, None) == INVALID
    assert g2(P, P, 0, 16, 0, 256, 128, _w(), P * 64, None, 0, None) == INVALID
    u = L.moe_fused_experts_unfinalized
    # deferred batched: R_pad must hold E_l * capacity rows
    assert u(P, P, 16, 128, 256, 8, 8, 2, 0, 1, 1.0, None, _w(), _w(), _opts(batched=16), 127,
             P, P, P, P, 1 << 30, None) == SIZE


def test_fp8_errors(L):
    q = L.moe_quantize_fp8
    # (x, rows, H, static, row_weights, row_count, q, scales, stream)
    assert q(P, 4, 120, None, None, None, P * 64, P * 128, None) == INVALID   # H % 16
    assert q(P, -1, 128, None, None, None, P * 64, P * 128, None) == INVALID
    assert q(P, 4, 128, P + 2, None, None, P * 64, P * 128, None) == MISALIGNED
    assert q(P, 4, 128, None, None, None, P + 256, P * 128, None) == CONFLICT  # q inside x
    assert q(P, 0, 128, None, None, None, None, None, None) == OK
    FP8 = 3
    g1 = L.moe_grouped_gemm1_act_fp8
    # (a, a_scales, offsets, E_l, R_pad, H, I, w1, act, clamp, h, ws, wsb, stream)
    assert g1(P, P, P, 8, 128, 128, 256, _w(), 0, 0.0, P * 64, None, 0, None) == INVALID  # bf16 w
    assert g1(P, P, P, 8, 128, 192, 256, _w(FP8, P, P), 0, 0.0, P * 64, None, 0, None) == INVALID
    assert g1(P, None, P, 8, 128, 128, 256, _w(FP8, P, P), 0, 0.0, P * 64, None, 0, None) == INVALID
    assert g1(P, P, P, 8, 128, 128, 256, _w(FP8, P, None), 0, 0.0, P * 64, None, 0, None) == INVALID
    # FP8 weights with bf16 activations
    assert L.moe_grouped_gemm1_act(P, P, 8, 128, 128, 256, _w(FP8, P, P), 0, 0.0, P * 64, None,
                                   0, None) == INVALID
    assert b"FP8 activations" in L.moe_last_error()
    g2 = L.moe_grouped_gemm2_fp8
    assert g2(P, P, P, 8, 128, 256, 128, _w(), P * 64, None, 0, None) == INVALID
    pf = L.moe_permute_fp8
    # (ids, emap, T, k, E, E_l, xq, xs, H, R_pad, map, offsets, inv, xq_perm, ps, stream)
    assert pf(P, None, 16, 2, 8, 8, P, P, 120, 32, P, P, None, P * 64, P * 128, None) == INVALID
    assert pf(P, None, 16, 2, 8, 8, P, P, 128, 31, P, P, None, P * 64, P * 128, None) == SIZE
    assert pf(P, None, 16, 2, 8, 8, P, None, 128, 32, P, P, None, P * 64, P * 128, None) == INVALID
    assert pf(P, None, 16, 2, 8, 8, P, P, 128, 32, P, P, None, P + 1024, P * 128, None) == CONFLICT
    u = L.moe_fused_experts_unfinalized

    def call(w=_w(FP8, P, P), opts=None, T=16, H=128, I=256):
        return u(P, P, T, H, I, 8, 8, 2, 0, 1, 1.0, None, w, w, opts, 32, P, P, P, P, 1 << 30, None)
    # FP8 in the batched layout: R_pad must hold E_l * capacity rows
    assert call(opts=_opts(quant=1, batched=16)) == SIZE
    # blockwise FP8: block-scaled weights only, both ways
    assert call(opts=_opts(quant=3)) == INVALID                     # per-channel FP8 weights
    assert call(w=_w(4, P, P), opts=_opts(quant=1)) == INVALID       # block weights, per-row acts
    assert call(w=_w(4, P, P), opts=_opts(quant=3), H=192) == INVALID  # H not a multiple of 128
    assert call(opts=_opts(quant=7)) == UNSUPPORTED
    assert call(w=_w(), opts=_opts(quant=1)) == INVALID          # bf16 weights
    assert call(opts=None) == INVALID                            # FP8 weights, no quantization
    assert call(w=_w(), opts=_opts(a1=P)) == INVALID             # a static scale without FP8
    assert call(opts=_opts(quant=1), H=192) == INVALID           # H % 128
    assert call(opts=_opts(quant=1, a1=P + 2)) == MISALIGNED
    assert call(opts=_opts(quant=1), T=0) == OK
    n0, n1 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert L.moe_workspace_size(64, 8, 256, 256, 7168, 2048, FP8, 0, None, ctypes.byref(n0)) == OK
    assert L.moe_workspace_size(64, 8, 256, 256, 7168, 2048, FP8, 0, _opts(quant=1),
                                ctypes.byref(n1)) == OK
    assert n1.value >= n0.value + 64 * 7168 + 512 * 2048


def test_grouped_gemm_workspace_size():
    L = _lib.lib()
    n = ctypes.c_size_t(0)
    # the larger of: decode sizes' fp32 slices of R_pad x N_total (up to 16
    # within 64 MiB, after a 256-byte header), and the tail round's 256 fp32
    # slabs of a 128 x 256 tile (after a 1 KiB header)
    tail = 1024 + 256 * 128 * 256 * 4
    assert L.moe_grouped_gemm_workspace_size(128, 2048, 1, ctypes.byref(n)) == 0
    assert n.value == max(256 + 16 * 128 * 4096 * 4, tail)
    assert L.moe_grouped_gemm_workspace_size(512, 7168, 0, ctypes.byref(n)) == 0
    assert n.value == 256 + 4 * 512 * 7168 * 4
    # prefill sizes never split the reduction of every tile: the tail slabs only
    assert L.moe_grouped_gemm_workspace_size(16384, 2048, 1, ctypes.byref(n)) == 0
    assert n.value == tail
    assert L.moe_grouped_gemm_workspace_size(70000, 64, 0, ctypes.byref(n)) == 0
    assert n.value == tail
    assert L.moe_grouped_gemm_workspace_size(128, 100, 0, ctypes.byref(n)) == INVALID
    assert L.moe_grouped_gemm_workspace_size(128, 64, 0, None) == INVALID


def test_noalloc_host_checks(L):
    """The entry point on the static scratch checks on the host: a problem
    whose scratch exceeds the static array is rejected before any HIP call."""
    u = L.moe_fused_experts_unfinalized_noalloc
    args = dict(logits=P, x=P, T=8192, H=7168, I=2048, E=8, El=8, k=8, score=1, renorm=1,
                rsf=1.0, emap=None, w1=_w(), w2=_w(), opts=None, R_pad=65536, y=P, w=P, m=P,
                s=None)

    def call(**kw):
        a = dict(args, **kw)
        return u(*a.values())
    assert call() == SIZE
    assert b"static scratch" in L.moe_last_error()
    assert call(T=-1) == INVALID
    assert call(R_pad=100) == SIZE           # R_pad < T * k
    assert call(T=0, R_pad=0) == OK
    assert call(w1=_w(7, P, P)) == UNSUPPORTED
