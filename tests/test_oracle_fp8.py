"""Pins of the oracle's FP8 E4M3 path (quantized activations of vLLM's
modular_kernel.py prepare/apply: quant_dtype, per_act_token_quant, a1_scale,
a2_scale, w1_scale, w2_scale).

- the decode table equals torch's float8_e4m3fn (a library type) for all 256
  codes, and the format's landmark values (448, 2^-6, 2^-9, 1, NaN, -0);
- the encoder equals torch's round-to-nearest-even cast on random values
  across the whole range, on every midpoint between neighbouring codes (ties
  to the even code) and round-trips every code;
- per-row quantization: the largest element maps to 448, every element is
  within half a step of its code, zero rows give zero codes and scale 1, a
  static scale equals torch's cast of x / scale;
- the FP8 layer with one expert equals torch's MLP on the decoded rows.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import configs

F8 = torch.float8_e4m3fn


def _torch_decode(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(codes.astype(np.uint8)).view(F8).to(torch.float64).numpy()


def _torch_encode(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(F8).view(torch.uint8).numpy()


def test_decode_table_matches_torch_and_landmarks():
    codes = np.arange(256, dtype=np.uint8)
    ours = np.array([oracle.e4m3_decode(int(c)) for c in codes])
    ref = _torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert oracle.e4m3_decode(0x7E) == 448.0
    assert oracle.e4m3_decode(0x08) == 2.0 ** -6
    assert oracle.e4m3_decode(0x01) == 2.0 ** -9
    assert oracle.e4m3_decode(0x38) == 1.0
    assert np.isnan(oracle.e4m3_decode(0x7F)) and np.isnan(oracle.e4m3_decode(0xFF))
    assert np.signbit(oracle.e4m3_decode(0x80))


def test_encode_matches_torch_cast():
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.uniform(-448, 448, 4000), rng.normal(0, 1, 4000),
                        rng.normal(0, 2.0 ** -7, 2000)]).astype(np.float32)
    ours = np.array([oracle.e4m3_encode(float(x)) for x in v], dtype=np.uint8)
    assert np.array_equal(ours, _torch_encode(v))


def test_midpoints_round_to_even_and_codes_round_trip():
    for c in range(0x7E):  # positive finite codes below 448
        lo, hi = oracle.e4m3_decode(c), oracle.e4m3_decode(c + 1)
        mid = (lo + hi) / 2
        want = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(mid) == want, hex(c)
        assert oracle.e4m3_encode(-mid) == want | 0x80
        assert oracle.e4m3_encode(lo) == c
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(1e6) == 0x7E          # saturates
    assert _torch_encode(np.array([mid]))[0] == want


def test_quantize_rows_dynamic_and_static():
    x = synth.normal_bf16(71, 0, (24, 96))
    x[5] = 0  # an all-zero row
    q, sc = oracle.quantize_fp8_rows(x)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    deq = _torch_decode(q) * sc[:, None].astype(np.float64)
    for r in range(x.shape[0]):
        if r == 5:
            assert np.all(q[r] == 0) and sc[r] == 1.0
            continue
        amax = np.abs(xf[r]).max()
        assert np.float32(sc[r]) == np.float32(np.float32(amax) / np.float32(448.0))
        assert np.max(_torch_decode(q[r]) * np.sign(xf[r])) == 448.0
        # within half a step: 2^-4 relative for normals, 2^-10 * scale absolute below
        err = np.abs(deq[r] - xf[r])
        bound = np.maximum(np.abs(xf[r]) * 2.0 ** -4, 2.0 ** -10 * sc[r]) * 1.0001
        assert np.all(err <= bound)
    qs, ss = oracle.quantize_fp8_rows(x, static_scale=0.0125)
    assert np.all(ss == np.float32(0.0125))
    inv = np.float32(1.0) / np.float32(0.0125)
    v = np.clip((xf.astype(np.float32) * inv).astype(np.float32), -448, 448)
    assert np.array_equal(qs, _torch_encode(v))


def _fp8_weights(w_bf16):
    """Per-row FP8 weights from bf16 rows: torch's cast of w / (amax / 448)."""
    wf = synth.bf16_bits_to_f32(w_bf16).astype(np.float32)
    amax = np.abs(wf).max(axis=-1, keepdims=True)
    sc = (amax / np.float32(448.0)).astype(np.float32)
    q = _torch_encode(np.clip(wf / sc, -448, 448))
    return q.reshape(w_bf16.shape), sc[..., 0]


def test_fp8_single_expert_layer_is_torch_mlp_on_decoded_rows():
    cfg = configs.MoeConfig("f", T=10, H=128, I=64, E=1, k=1, score=configs.SOFTMAX,
                            renormalize=True, rsf=1.0, seed=72)
    x, logits = configs.make_activations(cfg)
    w = configs.make_weights(cfg)
    q1, s1 = _fp8_weights(w["w1"])
    q2, s2 = _fp8_weights(w["w2"])
    r = oracle.moe_tokens(x, logits, oracle.Weights(q1[0], s1[0]), oracle.Weights(q2[0], s2[0]),
                          cfg.I, 1, oracle.SOFTMAX, True, 1.0, fp8=True)
    W1 = torch.from_numpy(_torch_decode(q1[0]) * s1[0][:, None].astype(np.float64))
    W2 = torch.from_numpy(_torch_decode(q2[0]) * s2[0][:, None].astype(np.float64))
    xq, xs = oracle.quantize_fp8_rows(x)
    X = torch.from_numpy(_torch_decode(xq) * xs[:, None].astype(np.float64))
    h = torch.nn.functional.silu(X @ W1[:cfg.I].T) * (X @ W1[cfg.I:].T)
    hb = h.to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    hq, hs = oracle.quantize_fp8_rows(hb)
    Hh = torch.from_numpy(_torch_decode(hq) * hs[:, None].astype(np.float64))
    ref = (Hh @ W2.T).numpy()
    np.testing.assert_allclose(r["out"], ref, rtol=1e-10, atol=1e-12)
    # the row helpers give the same rows
    eor = np.zeros(cfg.T, dtype=np.int32)
    hr = oracle.hidden_rows_fp8(xq, xs, oracle.Weights(q1, s1.reshape(-1)), eor, cfg.I)
    np.testing.assert_allclose(hr, h.numpy(), rtol=1e-12, atol=1e-14)
    yr = oracle.out_rows_fp8(hq, hs, oracle.Weights(q2, s2.reshape(-1)), eor, cfg.H)
    np.testing.assert_allclose(yr, ref, rtol=1e-12, atol=1e-14)
