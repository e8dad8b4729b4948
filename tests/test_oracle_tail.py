"""Pins of the oracle's fused tail (finalize + residual add + RMSNorm of the
new residual, per vLLM's MoEOutput contract: the next layer's RMSNorm is the
consumer that folds the open reduction into itself).

- the norm part equals torch's rms_norm (a library routine) on the new residual;
- RMSNorm is invariant to scaling its input (eps = 0), and with gamma = 1 every
  output row has root-mean-square 1 (eps = 0);
- the residual part equals residual + the finalize output, term by term
  (finalize itself is pinned in test_oracle_layer.py);
- a token with no local route gets the RMSNorm of its residual (plus shared).
"""
import numpy as np
import torch

import oracle
import synth

H = 96


def _case(T=6, k=3, E=5, seed=11):
    rng = np.random.default_rng(seed)
    logits = synth.normal_f32(seed, 1, (T, E))
    ids, w = oracle.route(logits, k, 0, True, 1.0)
    emap = np.array([0, -1, 1, 2, -1], dtype=np.int32)  # experts 1 and 4 not local
    m, off, _ = oracle.permute(ids, E, 3, emap)
    R = int(off[-1])
    y = synth.normal_bf16(seed, 2, (max(R, 1), H))
    res = synth.normal_bf16(seed, 3, (T, H))
    gamma = synth.normal_bf16(seed, 4, (H,), mean=1.0, std=0.1)
    shared = synth.normal_bf16(seed, 5, (T, H))
    return y, w, m, res, gamma, shared


def test_norm_part_equals_torch_rms_norm():
    y, w, m, res, gamma, shared = _case()
    r_out, out = oracle.finalize_add_rmsnorm(y, w, m, res, gamma, 1e-6, 0.7, shared)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(r_out), (H,),
                                       weight=torch.from_numpy(synth.bf16_bits_to_f32(gamma).astype(np.float64)),
                                       eps=1e-6)
    assert np.allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_residual_part_is_residual_plus_finalize():
    y, w, m, res, gamma, shared = _case(seed=12)
    r_out, _ = oracle.finalize_add_rmsnorm(y, w, m, res, gamma, 1e-6, 2.5, shared)
    fin = oracle.finalize(y, w, m, 2.5, shared)
    assert np.allclose(r_out, fin + synth.bf16_bits_to_f32(res).astype(np.float64), rtol=0, atol=1e-12)


def test_rmsnorm_scale_invariance_and_unit_rms():
    y, w, m, res, gamma, shared = _case(seed=13)
    one = synth.bf16_bits_to_f32(np.full(H, 0x3F80, dtype=np.uint16))
    assert np.all(one == 1.0)
    gamma1 = np.full(H, 0x3F80, dtype=np.uint16)
    _, out = oracle.finalize_add_rmsnorm(y, w, m, res, gamma1, 0.0, 1.0, shared)
    assert np.allclose(np.sqrt(np.mean(out * out, axis=1)), 1.0, rtol=1e-12)
    # doubling every input term doubles the new residual, which leaves the norm unchanged
    y2 = (synth.bf16_bits_to_f32(y) * 2).astype(np.float32).view(np.uint32) >> 16
    res2 = (synth.bf16_bits_to_f32(res) * 2).astype(np.float32).view(np.uint32) >> 16
    sh2 = (synth.bf16_bits_to_f32(shared) * 2).astype(np.float32).view(np.uint32) >> 16
    _, out2 = oracle.finalize_add_rmsnorm(y2.astype(np.uint16), w, m, res2.astype(np.uint16),
                                          gamma1, 0.0, 1.0, sh2.astype(np.uint16))
    assert np.allclose(out2, out, rtol=1e-12, atol=1e-12)


def test_token_without_local_routes_normalizes_its_residual():
    y, w, m, res, gamma, shared = _case(seed=14)
    m = m.copy()
    m[0, :] = -1
    r_out, out = oracle.finalize_add_rmsnorm(y, w, m, res, gamma, 1e-5, 1.0, None)
    r0 = synth.bf16_bits_to_f32(res[0]).astype(np.float64)
    assert np.array_equal(r_out[0], r0)
    g = synth.bf16_bits_to_f32(gamma).astype(np.float64)
    assert np.allclose(out[0], r0 / np.sqrt(np.mean(r0 * r0) + 1e-5) * g, rtol=1e-12)
