"""GPU parity of the small layer variants and of activation chunking against
the oracle (modular_kernel.py: activation() "gelu", forward()'s
apply_router_weight_on_input, inplace and activation chunking;
flashinfer_moe_ep.py: the activation_clamp of the fused SwiGLU epilogue).

- GEMM1 with GELU and with a clamp, on every tile shape and on the split
  path, against oracle.hidden_rows (bar 1e-2 relative Frobenius);
- the whole layer with GELU + clamp, and with the router weight on the input
  (top_k = 1, sigmoid weights below 1): fused, deferred + finalize, and the
  permute gather's scaled rows bit for bit against fp32 products rounded to
  bf16;
- chunked layers (ragged last chunk, with and without the shared expert)
  against the oracle on sampled tokens and against the one-pass layer;
- in place (out = x) bit-identical to the out-of-place result.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_scan_amd as moe
import oracle
import synth
from synth import configs

from gpu_util import (dev, dev_bf16, host_bf16_bits, host_f64, need_gpu, rel_fro,
                      sample_tokens, segments_of)

pytestmark = pytest.mark.gpu

TOL = 1e-2
NAN_BITS = 0x7FC0


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


ACT_CASES = [
    # name, counts per local expert, H, I, activation, clamp
    ("thin_gelu", [0, 1, 5, 33, 2, 0, 17, 40], 256, 192, "gelu", 0.0),
    ("wide_gelu_clamp", [70, 0, 130, 55], 384, 320, "gelu", 0.75),
    ("mid_silu_clamp", [300, 1, 420], 256, 448, "silu", 0.5),
    ("big_gelu", [700, 613], 512, 384, "gelu", 0.0),
    ("split_decode_silu_clamp", [1, 0, 2, 1, 0, 3], 1024, 512, "silu", 0.5),
    ("split_wide_gelu_clamp", [20, 30, 0, 16], 1024, 512, "gelu", 1.0),
]


@pytest.mark.parametrize("case", ACT_CASES, ids=[c[0] for c in ACT_CASES])
def test_gemm1_activation_and_clamp(case):
    name, counts, H, I, act, clamp = case
    E_l = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R_l = int(offsets[-1])
    R_pad = ((R_l + 127) // 128) * 128
    seed = sum(counts) + 31
    a = synth.normal_bf16(seed, 0, (R_pad, H))
    a[R_l:] = NAN_BITS
    w1 = synth.normal_bf16(seed, 2, (E_l, 2 * I, H), std=1 / np.sqrt(H))
    h = torch.full((R_pad, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm1_act(dev_bf16(a), dev(offsets), moe.Weights(dev_bf16(w1)), I, h=h,
                              activation=act, activation_clamp=clamp)
    torch.cuda.synchronize()
    eor = segments_of(offsets, R_l)
    ref = oracle.hidden_rows(a[:R_l], oracle.Weights(w1), eor, I, activation=act, clamp=clamp)
    assert rel_fro(host_f64(h, slice(None, R_l)), ref) < TOL
    assert np.all(host_bf16_bits(h)[R_l:] == NAN_BITS)
    if clamp:
        # the clamp was active: the unclamped oracle is far off
        plain = oracle.hidden_rows(a[:R_l], oracle.Weights(w1), eor, I, activation=act)
        assert rel_fro(plain, ref) > 5 * TOL


def _small_cfg(name, T, H, I, E, k, score, renorm, rsf, seed, shared_I=0):
    return configs.MoeConfig(name, T=T, H=H, I=I, E=E, k=k, score=score, renormalize=renorm,
                             rsf=rsf, seed=seed, shared_I=shared_I)


def _upload(cfg, w):
    d = {"w1": moe.Weights(dev_bf16(w["w1"])), "w2": moe.Weights(dev_bf16(w["w2"]))}
    if cfg.shared_I:
        d["ws1"], d["ws2"] = dev_bf16(w["ws1"]), dev_bf16(w["ws2"])
    return d


def _oracle(cfg, x, logits, w, tokens=None, **kw):
    return oracle.moe_tokens(x, logits, oracle.Weights(w["w1"]), oracle.Weights(w["w2"]), cfg.I,
                             cfg.k, cfg.score, cfg.renormalize, cfg.rsf, shared_I=cfg.shared_I,
                             ws1=w.get("ws1"), ws2=w.get("ws2"), tokens=tokens, **kw)


@pytest.mark.parametrize("act,clamp", [("gelu", 0.0), ("gelu", 0.75), ("silu", 0.5)])
def test_layer_activation_variants(act, clamp):
    cfg = _small_cfg("v", T=200, H=256, I=320, E=8, k=2, score=configs.SOFTMAX, renorm=True,
                     rsf=1.0, seed=41, shared_I=128)
    x, logits = configs.make_activations(cfg)
    w = configs.make_weights(cfg)
    W = _upload(cfg, w)
    out = moe.moe_fused_experts(dev(logits), dev_bf16(x), W["w1"], W["w2"], cfg.k, cfg.score,
                                cfg.renormalize, cfg.rsf, ws1=W["ws1"], ws2=W["ws2"],
                                activation=act, activation_clamp=clamp)
    y, ew, m = moe.moe_fused_experts_unfinalized(dev(logits), dev_bf16(x), W["w1"], W["w2"],
                                                 cfg.k, cfg.score, cfg.renormalize, cfg.rsf,
                                                 activation=act, activation_clamp=clamp)
    routed = moe.moe_finalize(y, ew, m)
    torch.cuda.synchronize()
    ref = _oracle(cfg, x, logits, w, activation=act, clamp=clamp)
    assert rel_fro(host_f64(out), ref["out"]) < TOL
    mm = m.cpu().numpy()
    yy = host_f64(y)
    assert rel_fro(yy[mm.reshape(-1)], ref["y_routes"].reshape(-1, cfg.H)) < TOL
    ref_routed = oracle.moe_tokens(x, logits, oracle.Weights(w["w1"]), oracle.Weights(w["w2"]),
                                   cfg.I, cfg.k, cfg.score, cfg.renormalize, cfg.rsf,
                                   activation=act, clamp=clamp)
    assert rel_fro(host_f64(routed), ref_routed["out"]) < TOL


def test_router_weight_on_input_top1():
    # sigmoid weights without renormalization stay below 1, so scaling the
    # input and scaling the output differ
    cfg = _small_cfg("w", T=300, H=256, I=192, E=8, k=1, score=configs.SIGMOID, renorm=False,
                     rsf=1.0, seed=42)
    x, logits = configs.make_activations(cfg)
    w = configs.make_weights(cfg)
    W = _upload(cfg, w)
    xd, ld = dev_bf16(x), dev(logits)
    out = moe.moe_fused_experts(ld, xd, W["w1"], W["w2"], 1, cfg.score, False, 1.0,
                                apply_router_weight_on_input=True)
    y, ew, m = moe.moe_fused_experts_unfinalized(ld, xd, W["w1"], W["w2"], 1, cfg.score, False,
                                                 1.0, apply_router_weight_on_input=True)
    fin = moe.moe_finalize(y, ew, m)
    fin_none = moe.moe_finalize(y, None, m)
    torch.cuda.synchronize()
    ref = _oracle(cfg, x, logits, w, weight_on_input=True)
    post = _oracle(cfg, x, logits, w)
    assert rel_fro(post["out"], ref["out"]) > 5 * TOL
    assert rel_fro(host_f64(out), ref["out"]) < TOL
    assert np.all(host_bf16_bits(ew) == 0x3F80)  # unit weights in the deferred triple
    assert rel_fro(host_f64(fin), ref["out"]) < TOL
    assert np.array_equal(host_bf16_bits(fin), host_bf16_bits(fin_none))
    assert np.array_equal(host_bf16_bits(fin), host_bf16_bits(out))


def test_permute_scales_gathered_rows_bit_exact():
    T, k, E, H = 37, 2, 6, 136
    logits = synth.normal_f32(43, 1, (T, E))
    ids, wts = moe.moe_route_topk(dev(logits), k, configs.SIGMOID, False, 1.0)
    x = synth.normal_bf16(43, 0, (T, H))
    p = moe.moe_permute(ids, E, x=dev_bf16(x), x_weights=wts)
    torch.cuda.synchronize()
    m = p["map"].cpu().numpy()
    w32 = wts.cpu().numpy()
    got = host_bf16_bits(p["x_perm"])
    xf = synth.bf16_bits_to_f32(x)
    for t in range(T):
        for j in range(k):
            prod = (np.float32(w32[t, j]) * xf[t]).astype(np.float32)
            u = prod.view(np.uint32).astype(np.uint64)
            want = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)  # RNE to bf16
            assert np.array_equal(got[m[t, j]], want), (t, j)


CHUNK_CASES = [
    # name, T, H, I, E, k, shared_I, chunk
    ("ragged_chunks", 1000, 512, 384, 8, 2, 0, 256),
    ("shared_expert_chunks", 300, 256, 256, 16, 4, 128, 128),
    ("one_token_chunks", 5, 128, 256, 8, 2, 64, 1),
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=[c[0] for c in CHUNK_CASES])
def test_chunked_layer(case):
    name, T, H, I, E, k, shared_I, chunk = case
    cfg = _small_cfg(name, T=T, H=H, I=I, E=E, k=k, score=configs.SOFTMAX, renorm=True,
                     rsf=1.0, seed=44 + T, shared_I=shared_I)
    x, logits = configs.make_activations(cfg)
    w = configs.make_weights(cfg)
    W = _upload(cfg, w)
    kw = dict(ws1=W["ws1"], ws2=W["ws2"]) if shared_I else {}
    xd, ld = dev_bf16(x), dev(logits)
    one = moe.moe_fused_experts(ld, xd, W["w1"], W["w2"], k, **kw)
    ws_chunk = moe.moe_workspace_size(T, k, E, E, H, I, shared_I=shared_I, chunk_tokens=chunk)
    assert ws_chunk == (moe.moe_workspace_size(chunk, k, E, E, H, I)
                        + moe.moe_shared_workspace_size(chunk, H, shared_I))
    ws = torch.empty(ws_chunk, dtype=torch.uint8, device="cuda")
    chunked = moe.moe_fused_experts(ld, xd, W["w1"], W["w2"], k, chunk_tokens=chunk,
                                    workspace=ws, **kw)
    again = moe.moe_fused_experts(ld, xd, W["w1"], W["w2"], k, chunk_tokens=chunk,
                                  workspace=ws, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(chunked), host_bf16_bits(again))
    assert rel_fro(host_f64(chunked), host_f64(one)) < TOL
    toks = sample_tokens(T, 40, 7)
    ref = _oracle(cfg, x, logits, w, tokens=toks)
    assert rel_fro(host_f64(chunked, toks), ref["out"]) < TOL


@pytest.mark.parametrize("chunk", [0, 96])
def test_in_place_equals_out_of_place(chunk):
    cfg = _small_cfg("ip", T=257, H=256, I=256, E=8, k=2, score=configs.SOFTMAX, renorm=True,
                     rsf=1.0, seed=45, shared_I=128)
    x, logits = configs.make_activations(cfg)
    w = configs.make_weights(cfg)
    W = _upload(cfg, w)
    ld = dev(logits)
    ref = moe.moe_fused_experts(ld, dev_bf16(x), W["w1"], W["w2"], cfg.k, ws1=W["ws1"],
                                ws2=W["ws2"], chunk_tokens=chunk)
    xd = dev_bf16(x)
    out = moe.moe_fused_experts(ld, xd, W["w1"], W["w2"], cfg.k, ws1=W["ws1"], ws2=W["ws2"],
                                chunk_tokens=chunk, inplace=True)
    torch.cuda.synchronize()
    assert out.data_ptr() == xd.data_ptr()
    assert np.array_equal(host_bf16_bits(out), host_bf16_bits(ref))
    o = _oracle(cfg, x, logits, w, tokens=sample_tokens(cfg.T, 20, 3))
    assert rel_fro(host_f64(out)[o["tokens"]], o["out"]) < TOL
