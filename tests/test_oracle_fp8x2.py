"""Pins of the oracle's two-term FP8 quantization (bf16 activations carried to
the FP8 x e2m1 matrix cores for MXFP4 weights: the quantize step of vLLM's
modular_kernel.py prepare; x ~ scale * (q1 + q2 / 16)).

- the first term and the scale are exactly the one-term per-row quantizer's
  (itself pinned against torch's float8_e4m3fn cast in test_oracle_fp8.py);
- the second term is torch's round-to-nearest-even cast of 16 times the
  residual, recomputed here with numpy float32 arithmetic and torch's
  decode, not with the oracle's encoder;
- the closed-form error bound of two E4M3 terms: |v - (q1 + q2 / 16)| <=
  2^-8 |v| + 2^-14 for v = x * 448 / amax, which the first term alone
  breaks, and which the data come close to (so a dropped or mis-scaled term
  fails it);
- rows whose scaled values are E4M3 values already give q2 = 0;
- the two-term layer with one expert and MXFP4 weights equals torch's MLP on
  the decoded rows, and is within bf16-like error of the plain bf16 layer.
"""
import numpy as np
import torch

import oracle
import synth
from synth import configs

F8 = torch.float8_e4m3fn


def _decode(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(codes.astype(np.uint8)).view(F8).to(torch.float64).numpy()


def _encode(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(F8).view(torch.uint8).numpy()


def _rows(seed=11, rows=24, H=320):
    x = synth.normal_bf16(seed, 0, (rows, H))
    x[3] = 0                                  # an all-zero row
    x[5, :] = synth.normal_bf16(seed, 1, (H,), std=1e-3)  # a small-magnitude row
    return x


def test_first_term_and_scale_are_the_one_term_quantizer():
    x = _rows()
    q1, q2, sc = oracle.quantize_fp8x2_rows(x)
    q, s = oracle.quantize_fp8_rows(x)
    assert np.array_equal(q1, q) and np.array_equal(sc, s)
    assert np.all(q2[3] == 0) and sc[3] == np.float32(1.0)


def _scaled(x):
    """v = clamp(x * (448 / amax)) per row in float32 (amax 448 for a zero row)."""
    xf = synth.bf16_bits_to_f32(x)
    amax = np.abs(xf).max(axis=1)
    amax = np.where(amax == 0, np.float32(448.0), amax).astype(np.float32)
    inv = (np.float32(448.0) / amax).astype(np.float32)
    return np.clip((xf * inv[:, None]).astype(np.float32), -448, 448).astype(np.float32)


def test_second_term_is_the_cast_of_sixteen_times_the_residual():
    x = _rows(seed=12)
    q1, q2, sc = oracle.quantize_fp8x2_rows(x)
    v = _scaled(x)
    d = (v.astype(np.float64) - _decode(q1)).astype(np.float32)
    assert np.array_equal(d.astype(np.float64), v.astype(np.float64) - _decode(q1))  # exact
    assert np.array_equal(q2, _encode(np.float32(16.0) * d))


def test_two_term_error_bound_is_met_and_nearly_tight():
    x = _rows(seed=13, rows=64, H=512)
    q1, q2, sc = oracle.quantize_fp8x2_rows(x)
    v = _scaled(x).astype(np.float64)
    two = _decode(q1) + _decode(q2) / 16.0
    err = np.abs(v - two)
    bound = 2.0 ** -8 * np.abs(v) + 2.0 ** -14
    assert np.all(err <= bound)
    assert np.any(np.abs(v - _decode(q1)) > bound)   # the first term alone is not enough
    big = np.abs(v) > 1.0
    assert np.max(err[big] / np.abs(v[big])) > 2.0 ** -11   # close to the bound's order
    # reconstruction of x itself, relative to the row norm
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    rel = np.linalg.norm(xf - two * sc[:, None], axis=1) / np.maximum(
        np.linalg.norm(xf, axis=1), 1e-30)
    assert np.all(rel < 2.0 ** -8)


def test_exact_e4m3_rows_have_zero_second_term():
    codes = np.arange(0, 0x7F, dtype=np.uint8)  # all non-negative finite codes
    vals = np.concatenate([_decode(codes), -_decode(codes)])
    vals[0] = 448.0                              # amax 448: inv = 1, v = x
    bits = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
    x = bits.numpy().view(np.uint16)[None, :]
    assert np.array_equal(synth.bf16_bits_to_f32(x)[0].astype(np.float64), vals)  # exact in bf16
    q1, q2, sc = oracle.quantize_fp8x2_rows(x)
    assert sc[0] == np.float32(1.0)
    assert np.array_equal(_decode(q1[0]), vals)
    assert np.all(q2 == 0)


def test_two_term_single_expert_layer_is_torch_mlp_on_decoded_rows():
    cfg = configs.MoeConfig("x2", T=12, H=256, I=256, E=1, k=1, score=configs.SOFTMAX,
                            renormalize=True, rsf=1.0, seed=73, mxfp4=True)
    x, logits = configs.make_activations(cfg)
    w = configs.make_weights(cfg)
    W1q, W2q = oracle.Weights(w["w1_q"], w["w1_s"]), oracle.Weights(w["w2_q"], w["w2_s"])
    r = oracle.moe_tokens(x, logits, W1q, W2q, cfg.I, 1, oracle.SOFTMAX, True, 1.0, fp8="x2")
    W1 = torch.from_numpy(oracle.mxfp4_dequant(w["w1_q"][0], w["w1_s"][0]))
    W2 = torch.from_numpy(oracle.mxfp4_dequant(w["w2_q"][0], w["w2_s"][0]))
    a1, a2, sa = oracle.quantize_fp8x2_rows(x)
    X = torch.from_numpy((_decode(a1) + _decode(a2) / 16.0) * sa[:, None].astype(np.float64))
    h = torch.nn.functional.silu(X @ W1[:cfg.I].T) * (X @ W1[cfg.I:].T)
    hb = h.to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    b1, b2, sb = oracle.quantize_fp8x2_rows(hb)
    Hh = torch.from_numpy((_decode(b1) + _decode(b2) / 16.0) * sb[:, None].astype(np.float64))
    ref = (Hh @ W2.T).numpy()
    np.testing.assert_allclose(r["out"], ref, rtol=1e-10, atol=1e-12)
    plain = oracle.moe_tokens(x, logits, W1q, W2q, cfg.I, 1, oracle.SOFTMAX, True, 1.0)
    rel = np.linalg.norm(r["out"] - plain["out"]) / np.linalg.norm(plain["out"])
    assert rel < 1e-2


def test_two_term_row_helpers_are_torch_mlp_on_decoded_rows():
    rows, H, I = 9, 256, 256
    x = synth.normal_bf16(74, 0, (rows, H))
    hb = synth.normal_bf16(74, 1, (rows, I))
    w1q, w1s = synth.mxfp4_quantize(synth.normal_bf16(74, 2, (1, 2 * I, H), std=1 / 16))
    w2q, w2s = synth.mxfp4_quantize(synth.normal_bf16(74, 3, (1, H, I), std=1 / 16))
    W1 = torch.from_numpy(oracle.mxfp4_dequant(w1q[0], w1s[0]))
    W2 = torch.from_numpy(oracle.mxfp4_dequant(w2q[0], w2s[0]))
    a1, a2, sa = oracle.quantize_fp8x2_rows(x)
    b1, b2, sb = oracle.quantize_fp8x2_rows(hb)
    X = torch.from_numpy((_decode(a1) + _decode(a2) / 16.0) * sa[:, None].astype(np.float64))
    Hh = torch.from_numpy((_decode(b1) + _decode(b2) / 16.0) * sb[:, None].astype(np.float64))
    eor = np.zeros(rows, dtype=np.int32)
    h = oracle.hidden_rows_fp8x2(a1, a2, sa, oracle.Weights(w1q, w1s), eor, I)
    ref_h = torch.nn.functional.silu(X @ W1[:I].T) * (X @ W1[I:].T)
    np.testing.assert_allclose(h, ref_h.numpy(), rtol=1e-12, atol=1e-14)
    y = oracle.out_rows_fp8x2(b1, b2, sb, oracle.Weights(w2q, w2s), eor, H)
    np.testing.assert_allclose(y, (Hh @ W2.T).numpy(), rtol=1e-12, atol=1e-14)
