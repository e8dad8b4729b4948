"""Pins of the oracle's block-scaled FP8 path (vLLM modular_kernel.py,
FusedMoEPermuteExpertsUnpermute quant properties: block_shape and
per_act_token_quant; weights with one scale per 128 x 128 block, activations
with one scale per token and group of 128 elements).

- the group quantizer equals the pinned per-row quantizer run on each group
  alone, and torch's float8_e4m3fn cast of x * 448 / amax(group);
- a layer of two experts with block-scaled weights (4 x 2 blocks per GEMM1
  matrix, 2 x 4 per GEMM2 matrix, every block its own scale) and group-scaled
  activations equals the same mixture computed by torch from the decoded
  values (torch's FP8 decode times the repeated scales), so a transposed,
  shifted or per-expert-misplaced block index fails;
- the row helpers with [rows, K/128] scales give the same hidden and output
  rows.
"""
import numpy as np
import torch

import oracle
import synth
from synth import configs

F8 = torch.float8_e4m3fn


def _dec(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(F8).to(
        torch.float64).numpy()


def test_group_quantizer_is_row_quantizer_per_group_and_torch_cast():
    x = synth.normal_bf16(140, 0, (6, 512), std=2.0)
    x[2, 128:256] = 0                              # an all-zero group
    q, s = oracle.quantize_fp8_groups(x)
    assert q.shape == (6, 512) and s.shape == (6, 4)
    qr, sr = oracle.quantize_fp8_rows(np.ascontiguousarray(x.reshape(-1, 128)))
    assert np.array_equal(q, qr.reshape(6, 512))
    assert np.array_equal(s.reshape(-1).view(np.uint32), sr.view(np.uint32))
    xf = synth.bf16_bits_to_f32(x).reshape(6, 4, 128)
    amax = np.abs(xf).max(axis=-1)
    amax = np.where(amax == 0, np.float32(448.0), amax).astype(np.float32)
    inv = (np.float32(448.0) / amax).astype(np.float32)
    v = np.clip((xf * inv[..., None]).astype(np.float32), -448, 448)
    want = torch.from_numpy(v).to(F8).view(torch.uint8).numpy().reshape(6, 512)
    assert np.array_equal(q, want)
    assert s[2, 1] == 1.0 and np.all(q[2, 128:256] == 0)


def _deq_blocks(q, s):
    return _dec(q) * np.repeat(np.repeat(s.astype(np.float64), 128, -2), 128, -1)


def test_block_layer_is_torch_mixture_on_decoded_values():
    cfg = configs.MoeConfig("fb", T=7, H=256, I=256, E=2, k=2, score=configs.SOFTMAX,
                            renormalize=True, rsf=1.0, seed=141)
    x, logits = configs.make_activations(cfg)
    w = configs.make_weights(cfg)
    q1, s1 = synth.fp8_quantize_blocks(w["w1"])      # [2, 512, 256], [2, 4, 2]
    q2, s2 = synth.fp8_quantize_blocks(w["w2"])      # [2, 256, 256], [2, 2, 2]
    assert len(np.unique(s1)) == s1.size             # every block its own scale
    W1o = oracle.Weights(q1, s1, block=True)
    W2o = oracle.Weights(q2, s2, block=True)
    r = oracle.moe_tokens(x, logits, W1o, W2o, cfg.I, cfg.k, cfg.score, True, 1.0, fp8="block")
    W1, W2 = _deq_blocks(q1, s1), _deq_blocks(q2, s2)
    xq, xs = oracle.quantize_fp8_groups(x)
    X = _dec(xq) * np.repeat(xs.astype(np.float64), 128, -1)
    p = torch.softmax(torch.from_numpy(logits.astype(np.float64)), dim=-1).numpy()
    ref = np.zeros((cfg.T, cfg.H))
    rows_h, rows_y = [], []
    for e in range(cfg.E):                         # k = E: every expert on every token
        Wt = torch.from_numpy(W1[e])
        g = torch.from_numpy(X) @ Wt[:cfg.I].T
        u = torch.from_numpy(X) @ Wt[cfg.I:].T
        h = torch.nn.functional.silu(g) * u
        hb = h.to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        hq, hs = oracle.quantize_fp8_groups(hb)
        Hd = _dec(hq) * np.repeat(hs.astype(np.float64), 128, -1)
        y = Hd @ W2[e].T
        ref += p[:, e:e + 1] * y
        rows_h.append((h.numpy(), hq, hs, y))
    np.testing.assert_allclose(r["out"], ref, rtol=1e-10, atol=1e-12)
    # the row helpers on group-scaled rows, expert 1 (block rows 4..7 / 2..3)
    eor = np.ones(cfg.T, dtype=np.int32)
    h1, hq1, hs1, y1 = rows_h[1]
    np.testing.assert_allclose(oracle.hidden_rows_fp8(xq, xs, W1o, eor, cfg.I), h1,
                               rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(oracle.out_rows_fp8(hq1, hs1, W2o, eor, cfg.H), y1,
                               rtol=1e-12, atol=1e-14)
