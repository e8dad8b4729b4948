"""Pins of the oracle's small layer variants (modular_kernel.py: activation()
with "gelu", forward() with apply_router_weight_on_input; flashinfer_moe_ep.py:
the activation_clamp of the fused SwiGLU epilogue).

- GELU: the erf form, against torch's exact gelu (a library routine) on the
  single-expert layer and on rows; the standard normal CDF at 1 printed to 16
  digits (gelu(1) = Phi(1)), which the tanh approximation misses by 1.5e-4.
- clamp: hand-worked gate/up values built from one-hot rows; a clamp above
  every |gate| and |up| changes nothing.
- router weight on the input (top_k = 1): equals torch's MLP of the scaled
  token for the argmax expert with the sigmoid weight; with softmax
  renormalized over one expert the weight is exactly 1 and nothing changes.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import configs

ONE = 0x3F80  # bf16 1.0


def _f64(bits):
    return torch.from_numpy(synth.bf16_bits_to_f32(bits).astype(np.float64))


def _bf16(values):
    """Exact bf16 bit patterns of small float values (each exactly representable)."""
    f = np.asarray(values, dtype=np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(synth.bf16_bits_to_f32(b), f)
    return b


def _glu_mlp(x, w1, w2, act):
    I = w2.shape[1]
    return (act(x @ w1[:I].T) * (x @ w1[I:].T)) @ w2.T


def _gelu(v):
    return torch.nn.functional.gelu(v, approximate="none")


def _tiny(seed, T=12, H=64, I=128, E=4):
    cfg = configs.MoeConfig("t", T=T, H=H, I=I, E=E, k=1, score=configs.SOFTMAX,
                            renormalize=True, rsf=1.0, seed=seed)
    x, logits = configs.make_activations(cfg)
    w = configs.make_weights(cfg)
    return cfg, x, logits, w


def test_gelu_single_expert_is_textbook_geglu():
    cfg, x, logits, w = _tiny(seed=21, E=1)
    r = oracle.moe_tokens(x, logits, oracle.Weights(w["w1"]), oracle.Weights(w["w2"]), cfg.I,
                          k=1, score=oracle.SOFTMAX, renormalize=True, rsf=1.0,
                          activation="gelu")
    ref = _glu_mlp(_f64(x), _f64(w["w1"][0]), _f64(w["w2"][0]), _gelu).numpy()
    np.testing.assert_allclose(r["out"], ref, rtol=1e-11, atol=1e-12)


def test_gelu_hidden_rows_match_torch():
    cfg, x, logits, w = _tiny(seed=22, E=3)
    eor = np.arange(cfg.T, dtype=np.int32) % 3
    h = oracle.hidden_rows(x, oracle.Weights(w["w1"]), eor, cfg.I, activation="gelu")
    xs = _f64(x)
    for r in range(cfg.T):
        W = _f64(w["w1"][eor[r]])
        ref = _gelu(xs[r] @ W[:cfg.I].T) * (xs[r] @ W[cfg.I:].T)
        np.testing.assert_allclose(h[r], ref.numpy(), rtol=1e-12, atol=1e-14)


def _one_hot_rows(H, I, gates, ups):
    """x = e_0 and w1 rows gate_i = gates[i] e_0, up_i = ups[i] e_0, so that
    g_i = gates[i] and u_i = ups[i] exactly."""
    x = np.zeros((1, H), dtype=np.uint16)
    x[0, 0] = ONE
    w1 = np.zeros((1, 2 * I, H), dtype=np.uint16)
    w1[0, :I, 0] = _bf16(gates)
    w1[0, I:, 0] = _bf16(ups)
    return x, w1


def test_gelu_of_one_is_the_normal_cdf():
    x, w1 = _one_hot_rows(64, 2, [1.0, 0.0], [1.0, 1.0])
    h = oracle.hidden_rows(x, oracle.Weights(w1), np.zeros(1, np.int32), 2, activation="gelu")
    assert abs(h[0, 0] - 0.8413447460685429) < 1e-15   # Phi(1), standard normal CDF
    assert h[0, 1] == 0.0


def test_clamp_hand_worked():
    # gates 5 (clamped to 2), -5 (below: untouched), 1; ups -3 (to -2), 1.5, 4 (to 2)
    x, w1 = _one_hot_rows(64, 3, [5.0, -5.0, 1.0], [-3.0, 1.5, 4.0])
    h = oracle.hidden_rows(x, oracle.Weights(w1), np.zeros(1, np.int32), 3, clamp=2.0)
    silu2 = 1.7615941559557649    # 2 / (1 + e^-2)
    silu_m5 = -0.03346425462142428  # -5 / (1 + e^5)
    silu1 = 0.7310585786300049    # 1 / (1 + e^-1)
    np.testing.assert_allclose(h[0], [silu2 * -2.0, silu_m5 * 1.5, silu1 * 2.0], rtol=1e-15)
    # without the clamp the same rows give the raw products
    h0 = oracle.hidden_rows(x, oracle.Weights(w1), np.zeros(1, np.int32), 3)
    assert abs(h0[0, 2] - silu1 * 4.0) < 1e-15


@pytest.mark.parametrize("activation", ["silu", "gelu"])
def test_clamp_above_every_value_changes_nothing(activation):
    cfg, x, logits, w = _tiny(seed=23, E=2)
    eor = np.arange(cfg.T, dtype=np.int32) % 2
    W = oracle.Weights(w["w1"])
    plain = oracle.hidden_rows(x, W, eor, cfg.I, activation=activation)
    big = oracle.hidden_rows(x, W, eor, cfg.I, activation=activation, clamp=1e6)
    assert np.array_equal(plain, big)
    small = oracle.hidden_rows(x, W, eor, cfg.I, activation=activation, clamp=0.25)
    assert not np.array_equal(plain, small)


def test_router_weight_on_input_top1_sigmoid():
    cfg, x, logits, w = _tiny(seed=24, E=4)
    r = oracle.moe_tokens(x, logits, oracle.Weights(w["w1"]), oracle.Weights(w["w2"]), cfg.I,
                          k=1, score=oracle.SIGMOID, renormalize=False, rsf=1.0,
                          weight_on_input=True)
    lt = torch.from_numpy(logits).double()
    xs = _f64(x)
    for t in range(cfg.T):
        e = int(torch.argmax(lt[t]))
        wt = torch.sigmoid(lt[t, e])
        ref = _glu_mlp(wt * xs[t:t + 1], _f64(w["w1"][e]), _f64(w["w2"][e]),
                       torch.nn.functional.silu).numpy()[0]
        assert r["ids"][t, 0] == e
        np.testing.assert_allclose(r["out"][t], ref, rtol=1e-11, atol=1e-13)
    # the weight really moved inside: the post-weighted layer differs
    post = oracle.moe_tokens(x, logits, oracle.Weights(w["w1"]), oracle.Weights(w["w2"]),
                             cfg.I, k=1, score=oracle.SIGMOID, renormalize=False, rsf=1.0)
    assert not np.allclose(post["out"], r["out"])


def test_router_weight_on_input_with_unit_weights_is_a_no_op():
    cfg, x, logits, w = _tiny(seed=25, E=4)
    args = (x, logits, oracle.Weights(w["w1"]), oracle.Weights(w["w2"]), cfg.I)
    kw = dict(k=1, score=oracle.SOFTMAX, renormalize=True, rsf=1.0)
    a = oracle.moe_tokens(*args, **kw, weight_on_input=True)
    b = oracle.moe_tokens(*args, **kw)
    assert np.all(b["weights"] == 1.0)
    assert np.array_equal(a["out"], b["out"])


def test_shared_expert_takes_the_layer_activation():
    cfg, x, logits, w = _tiny(seed=26, E=1)
    I_s = 64
    ws1 = synth.normal_bf16(26, 4, (2 * I_s, cfg.H), std=1 / np.sqrt(cfg.H))
    ws2 = synth.normal_bf16(26, 5, (cfg.H, I_s), std=1 / np.sqrt(I_s))
    r = oracle.moe_tokens(x, logits, oracle.Weights(w["w1"]), oracle.Weights(w["w2"]), cfg.I,
                          k=1, score=oracle.SOFTMAX, renormalize=True, rsf=1.0, shared_I=I_s,
                          ws1=ws1, ws2=ws2, activation="gelu")
    xs = _f64(x)
    ref = (_glu_mlp(xs, _f64(w["w1"][0]), _f64(w["w2"][0]), _gelu)
           + _glu_mlp(xs, _f64(ws1), _f64(ws2), _gelu)).numpy()
    np.testing.assert_allclose(r["out"], ref, rtol=1e-11, atol=1e-12)
