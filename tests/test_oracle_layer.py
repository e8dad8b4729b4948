"""Pins of the oracle's expert MLP, finalize and whole-layer composition.

- E=1, k=1 and top_k=1: the layer reduces to the textbook SiLU-gated MLP
  (silu(x Wg^T) * (x Wu^T)) W2^T, computed here with torch in float64.
- The dense mixture sum_e G[t,e] MLP_e(x_t) over *all* experts, with G zero
  off the top-k (torch softmax/topk), equals the oracle's per-route result.
- -1 routes contribute nothing; finalize is linear in the weights; rows the
  map never names are never read (NaN there changes nothing).
- MXFP4 weights give the same layer as bf16 weights holding the decoded values.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import configs


def _f64(bits):
    return torch.from_numpy(synth.bf16_bits_to_f32(bits).astype(np.float64))


def _swiglu(x, w1, w2):
    """Textbook SiLU-gated MLP in float64: x [n,H], w1 [2I,H], w2 [H,I]."""
    I = w2.shape[1]
    g = x @ w1[:I].T
    u = x @ w1[I:].T
    return (torch.nn.functional.silu(g) * u) @ w2.T


def _tiny(seed=1, T=16, H=128, I=256, E=8):
    cfg = configs.MoeConfig("t", T=T, H=H, I=I, E=E, k=2, score=configs.SOFTMAX,
                            renormalize=True, rsf=1.0, seed=seed)
    x, logits = configs.make_activations(cfg)
    w = configs.make_weights(cfg)
    return cfg, x, logits, w


def test_single_expert_is_textbook_swiglu():
    cfg, x, logits, w = _tiny(E=1)
    r = oracle.moe_tokens(x, logits, oracle.Weights(w["w1"]), oracle.Weights(w["w2"]), cfg.I,
                          k=1, score=oracle.SOFTMAX, renormalize=True, rsf=1.0)
    ref = _swiglu(_f64(x), _f64(w["w1"][0]), _f64(w["w2"][0])).numpy()
    assert np.all(r["weights"] == 1.0)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-11, atol=1e-12)


def test_top1_equals_chosen_expert_mlp():
    cfg, x, logits, w = _tiny(seed=2)
    r = oracle.moe_tokens(x, logits, oracle.Weights(w["w1"]), oracle.Weights(w["w2"]), cfg.I,
                          k=1, score=oracle.SOFTMAX, renormalize=True, rsf=1.0)
    xs = _f64(x)
    for t in range(cfg.T):
        e = int(r["ids"][t, 0])
        ref = _swiglu(xs[t:t + 1], _f64(w["w1"][e]), _f64(w["w2"][e])).numpy()[0]
        np.testing.assert_allclose(r["out"][t], ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("score,rsf", [(configs.SOFTMAX, 1.0), (configs.SIGMOID, 2.5)])
def test_dense_mixture_brute_force(score, rsf):
    cfg, x, logits, w = _tiny(seed=3)
    k = 2
    r = oracle.moe_tokens(x, logits, oracle.Weights(w["w1"]), oracle.Weights(w["w2"]), cfg.I,
                          k=k, score=score, renormalize=True, rsf=rsf)
    lt = torch.from_numpy(logits).double()
    s = torch.softmax(lt, 1) if score == configs.SOFTMAX else torch.sigmoid(lt)
    top = torch.topk(lt, k, dim=1).indices
    G = torch.zeros_like(s)
    sel = torch.gather(s, 1, top)
    G.scatter_(1, top, rsf * sel / sel.sum(1, keepdim=True))
    xs = _f64(x)
    dense = torch.zeros(cfg.T, cfg.H, dtype=torch.float64)
    for e in range(cfg.E):
        dense += G[:, e:e + 1] * _swiglu(xs, _f64(w["w1"][e]), _f64(w["w2"][e]))
    np.testing.assert_allclose(r["out"], dense.numpy(), rtol=1e-10, atol=1e-12)


def test_shared_expert_add_and_rsf_fin():
    cfg, x, logits, w = _tiny(seed=4)
    Is = 64
    ws1 = synth.normal_bf16(4, synth.TID_WS1, (2 * Is, cfg.H), std=1 / np.sqrt(cfg.H))
    ws2 = synth.normal_bf16(4, synth.TID_WS2, (cfg.H, Is), std=1 / np.sqrt(Is))
    W1, W2 = oracle.Weights(w["w1"]), oracle.Weights(w["w2"])
    base = oracle.moe_tokens(x, logits, W1, W2, cfg.I, k=2, score=0, renormalize=True, rsf=1.0)
    both = oracle.moe_tokens(x, logits, W1, W2, cfg.I, k=2, score=0, renormalize=True, rsf=1.0,
                             shared_I=Is, ws1=ws1, ws2=ws2, rsf_fin=0.75)
    shared = _swiglu(_f64(x), _f64(ws1), _f64(ws2)).numpy()
    np.testing.assert_allclose(both["out"], 0.75 * base["out"] + shared, rtol=1e-11, atol=1e-12)


def test_nonlocal_routes_contribute_zero():
    cfg = configs.EP_DECODE
    T, H, I = 6, 64, 32
    small = configs.MoeConfig("t", T=T, H=H, I=I, E=cfg.E, k=8, score=configs.SIGMOID,
                              renormalize=True, rsf=2.5, seed=9, E_local=32, local_first=96)
    x, logits = configs.make_activations(small)
    w = configs.make_weights(small)
    emap = configs.expert_map(small)
    W1, W2 = oracle.Weights(w["w1"]), oracle.Weights(w["w2"])
    r = oracle.moe_tokens(x, logits, W1, W2, I, k=8, score=1, renormalize=True, rsf=2.5,
                          expert_map=emap)
    xs = _f64(x)
    for t in range(T):
        ref = np.zeros(H)
        for j in range(8):
            L = emap[r["ids"][t, j]]
            if L < 0:
                assert np.all(r["y_routes"][t, j] == 0.0)
                continue
            ref += r["weights"][t, j] * _swiglu(xs[t:t + 1], _f64(w["w1"][L]),
                                                _f64(w["w2"][L])).numpy()[0]
        np.testing.assert_allclose(r["out"][t], ref, rtol=1e-11, atol=1e-13)
    # a map with no local expert at all: output exactly zero (exactly shared)
    none = np.full(cfg.E, -1, dtype=np.int32)
    r0 = oracle.moe_tokens(x, logits, W1, W2, I, k=8, score=1, renormalize=True, rsf=2.5,
                           expert_map=none)
    assert np.all(r0["out"] == 0.0)


def _finalize_inputs(seed=7, T=12, k=3, H=40, E=5):
    logits = synth.normal_f32(seed, 1, (T, E))
    ids, w = oracle.route(logits, k, oracle.SOFTMAX, True, 1.0)
    emap = np.array([0, -1, 1, 2, -1], dtype=np.int32)
    m, off, _ = oracle.permute(ids, E=E, E_l=3, expert_map=emap)
    R_pad = 64
    y = synth.normal_bf16(seed, 2, (R_pad, H))
    return y, w, m, int(off[-1])


def test_finalize_matches_definition_and_is_linear():
    y, w, m, R_l = _finalize_inputs()
    out = oracle.finalize(y, w, m)
    yf = synth.bf16_bits_to_f32(y).astype(np.float64)
    T, k = m.shape
    for t in range(T):
        ref = sum(w[t, j] * yf[m[t, j]] for j in range(k) if m[t, j] >= 0)
        np.testing.assert_allclose(out[t], ref if np.ndim(ref) else np.zeros(y.shape[1]),
                                   rtol=1e-15, atol=0)
    np.testing.assert_allclose(oracle.finalize(y, 3.0 * w, m), 3.0 * out, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(oracle.finalize(y, w, m, rsf_fin=2.5), 2.5 * out, rtol=1e-14,
                               atol=0)


def test_finalize_one_hot_gathers_rows():
    y, w, m, R_l = _finalize_inputs(seed=8)
    one = np.zeros_like(w)
    one[:, 0] = 1.0
    out = oracle.finalize(y, one, m)
    yf = synth.bf16_bits_to_f32(y).astype(np.float64)
    for t in range(m.shape[0]):
        want = yf[m[t, 0]] if m[t, 0] >= 0 else np.zeros(y.shape[1])
        assert np.array_equal(out[t], want)


def test_finalize_never_reads_unreferenced_rows():
    y, w, m, R_l = _finalize_inputs(seed=9)
    clean = oracle.finalize(y, w, m)
    poisoned = y.copy()
    poisoned[R_l:] = 0x7FC0          # bf16 quiet NaN in every padding row
    assert np.array_equal(oracle.finalize(poisoned, w, m), clean)
    shared = synth.normal_bf16(9, 5, (m.shape[0], y.shape[1]))
    s = oracle.finalize(poisoned, w, m, shared_bf16=shared)
    np.testing.assert_allclose(s, clean + synth.bf16_bits_to_f32(shared), rtol=1e-15, atol=0)


def test_hidden_and_out_rows_match_torch():
    cfg, x, logits, w = _tiny(seed=10)
    eor = np.array([0, 3, 3, 7, 1, 0, 5, 2, 6, 4, 4, 1, 7, 2, 5, 6], dtype=np.int32)
    h = oracle.hidden_rows(x, oracle.Weights(w["w1"]), eor, cfg.I)
    xs = _f64(x)
    for r in range(cfg.T):
        W = _f64(w["w1"][eor[r]])
        ref = torch.nn.functional.silu(xs[r] @ W[:cfg.I].T) * (xs[r] @ W[cfg.I:].T)
        np.testing.assert_allclose(h[r], ref.numpy(), rtol=1e-12, atol=1e-14)
    hb = synth.normal_bf16(10, 7, (cfg.T, cfg.I))
    y = oracle.out_rows(hb, oracle.Weights(w["w2"]), eor, cfg.H)
    hs = _f64(hb)
    for r in range(cfg.T):
        ref = hs[r] @ _f64(w["w2"][eor[r]]).T
        np.testing.assert_allclose(y[r], ref.numpy(), rtol=1e-12, atol=1e-14)


def test_mxfp4_weights_equal_their_decoded_bf16_values():
    cfg, x, logits, w = _tiny(seed=11, T=6, H=64, I=64, E=4)
    q1, s1 = synth.mxfp4_quantize(w["w1"])
    q2, s2 = synth.mxfp4_quantize(w["w2"])

    def decoded_bf16(q, s):
        # the page's rule, written with numpy: LUT[nibble] * float(s << 23)
        lut = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6],
                       dtype=np.float32)
        vals = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), dtype=np.float32)
        vals[..., 0::2] = lut[q & 15]
        vals[..., 1::2] = lut[q >> 4]
        sf = (s.astype(np.uint32) << 23).view(np.float32)
        full = vals * np.repeat(sf, 32, axis=-1)
        return torch.from_numpy(full).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    a = oracle.moe_tokens(x, logits, oracle.Weights(q1, s1), oracle.Weights(q2, s2), 64, k=2,
                          score=0, renormalize=True, rsf=1.0)
    b = oracle.moe_tokens(x, logits, oracle.Weights(decoded_bf16(q1, s1)),
                          oracle.Weights(decoded_bf16(q2, s2)), 64, k=2, score=0,
                          renormalize=True, rsf=1.0)
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-13, atol=1e-15)
