"""The seeded input generator: published SplitMix64 vectors, determinism, and
the storage roundings (bf16 nearest-even, MXFP4 packing)."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import synth
from synth import configs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_ints(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [int(l) for l in f if l.strip() and not l.startswith("#")]


def test_splitmix64_published_vector():
    gamma = 0x9E3779B97F4A7C15
    want = _golden_ints("splitmix64_seed1234567.txt")
    got = [synth.splitmix64((1234567 + i * gamma) % (1 << 64)) for i in range(5)]
    assert got == want


def test_deterministic_and_stream_separated():
    a = synth.normal_f32(7, 0, (1000,))
    b = synth.normal_f32(7, 0, (1000,))
    c = synth.normal_f32(7, 1, (1000,))
    d = synth.normal_f32(8, 0, (1000,))
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)
    assert not np.array_equal(a, d)
    # element i is a pure function of (seed, tensor, i)
    for i in (0, 1, 517, 999):
        assert np.float32(synth.normal_at(7, 0, i)) == a[i]


def test_thread_count_independent():
    code = ("import numpy as np, synth; "
            "np.save('/dev/stdout', synth.normal_bf16(3, 2, (4096,)), allow_pickle=False)")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = []
    for nt in ("1", "5"):
        env = dict(os.environ, OMP_NUM_THREADS=nt, PYTHONPATH=root)
        outs.append(subprocess.check_output([sys.executable, "-c", code], env=env))
    assert outs[0] == outs[1]


def test_normal_moments():
    x = synth.normal_f32(11, 0, (1 << 20,)).astype(np.float64)
    assert abs(x.mean()) < 5e-3
    assert abs(x.std() - 1.0) < 5e-3
    # Gaussian tail mass beyond 2 sigma is 4.55 %
    assert abs(np.mean(np.abs(x) > 2.0) - 0.0455) < 2e-3


def test_bf16_is_nearest_even_of_f32():
    f = synth.normal_f32(5, 3, (1 << 16,), std=0.37)
    b = synth.normal_bf16(5, 3, (1 << 16,), std=0.37)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


def test_zipf_bias_gives_imbalance():
    cfg = configs.MIXTRAL.with_T(4096)
    bias = synth.zipf_log_bias(cfg.E, cfg.zipf_s)
    p = np.exp(bias)
    assert abs(p.sum() - 1.0) < 1e-12
    assert np.all(np.diff(p) < 0)
    assert abs(p[0] / p[1] - 2.0 ** 1.1) < 1e-12


def test_mxfp4_quantizer_packs_nearest_grid_value():
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    w = synth.normal_bf16(9, 2, (8, 64), std=0.05)
    q, s = synth.mxfp4_quantize(w)
    assert q.shape == (8, 32) and s.shape == (8, 2)
    wf = synth.bf16_bits_to_f32(w).astype(np.float64)
    for r in range(8):
        for b in range(2):
            blk = wf[r, b * 32:(b + 1) * 32]
            e = int(s[r, b]) - 127
            assert e == int(np.floor(np.log2(np.abs(blk).max()))) - 2
            for i in range(32):
                kk = b * 32 + i
                byte = q[r, kk // 2]
                code = (byte & 15) if kk % 2 == 0 else (byte >> 4)
                mag = grid[code & 7]
                scaled = abs(blk[i]) / 2.0 ** e
                best = np.min(np.abs(grid - min(scaled, 6.0)))
                assert abs(mag - min(scaled, 6.0)) == pytest.approx(best, abs=0)
                if mag != 0:
                    assert (code >= 8) == (blk[i] < 0)


def test_config_recipes():
    assert configs.permuted_rows(1, 8) == 128
    assert configs.permuted_rows(64, 8) == 512
    assert configs.permuted_rows(2048, 8) == 16384
    m = configs.expert_map(configs.EP_DECODE)
    assert m.shape == (256,) and m.dtype == np.int32
    assert np.array_equal(m[96:128], np.arange(32))
    assert np.sum(m >= 0) == 32 and np.all(m[m < 0] == -1)
    x, logits = configs.make_activations(configs.TINY)
    assert x.shape == (16, 128) and x.dtype == np.uint16
    assert logits.shape == (16, 8) and logits.dtype == np.float32
    w = configs.make_weights(configs.TINY)
    assert w["w1"].shape == (8, 512, 128) and w["w2"].shape == (8, 128, 256)
    w1f = synth.bf16_bits_to_f32(w["w1"]).astype(np.float64)
    assert abs(w1f.std() - 1 / np.sqrt(128)) < 2e-3


def test_fp8_weight_quantizer_per_row():
    import torch
    w = synth.normal_bf16(81, 2, (3, 16, 256), std=0.05)
    w[1, 4] = 0
    q, s = synth.fp8_quantize_rows(w)
    assert q.shape == w.shape and s.shape == w.shape[:-1]
    dec = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy() * s[..., None]
    wf = synth.bf16_bits_to_f32(w).astype(np.float64)
    assert np.all(q[1, 4] == 0) and s[1, 4] == 1.0
    assert np.all(np.abs(dec - wf) <= np.maximum(np.abs(wf) * 2.0 ** -4, 2.0 ** -10 * s[..., None]))
    top = np.abs(torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy())
    assert np.all(top.reshape(-1, 256)[np.arange(48) != 20].max(axis=1) == 448.0)
