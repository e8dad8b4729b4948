"""GPU parity of the whole layer against the oracle, on the five workloads.

- tiny layer: every token, through the fused entry point, through the
  individual calls, and in deferred form followed by a separate finalize;
- Mixtral-shaped prefill and DeepSeek-V3-shaped routed + shared layers at full
  size: ids, permute map and offsets of every token bit-exact; outputs of
  sampled tokens (the oracle runs one token at a time) within 1e-2 relative
  Frobenius error; the fused entry point bit-identical to the individual calls
  and to a second run;
- one expert-parallel rank's share at decode sizes 1, 8, 64 in deferred form:
  map bit-exact, valid gemm2_permuted rows and bf16 weights within 1e-2, then
  the separate finalize within 1e-2.
"""
import gc

import numpy as np
import pytest
import torch

import mixture_experts_layer_scan_amd as moe
import oracle
import synth
from synth import configs

from gpu_util import (dev, dev_bf16, host_bf16_bits, host_f64, need_gpu, rel_fro,
                      sample_tokens)

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _upload(cfg, w):
    if cfg.mxfp4:
        d = {"w1": moe.Weights(dev(w["w1_q"]), dev(w["w1_s"])),
             "w2": moe.Weights(dev(w["w2_q"]), dev(w["w2_s"]))}
    else:
        d = {"w1": moe.Weights(dev_bf16(w["w1"])), "w2": moe.Weights(dev_bf16(w["w2"]))}
    if cfg.shared_I:
        d["ws1"], d["ws2"] = dev_bf16(w["ws1"]), dev_bf16(w["ws2"])
    return d


def _oracle_weights(cfg, w):
    if cfg.mxfp4:
        return oracle.Weights(w["w1_q"], w["w1_s"]), oracle.Weights(w["w2_q"], w["w2_s"])
    return oracle.Weights(w["w1"]), oracle.Weights(w["w2"])


def _oracle(cfg, x, logits, w, tokens=None):
    W1, W2 = _oracle_weights(cfg, w)
    return oracle.moe_tokens(
        x, logits, W1, W2, cfg.I, cfg.k, cfg.score,
        cfg.renormalize, cfg.rsf, expert_map=configs.expert_map(cfg), shared_I=cfg.shared_I,
        ws1=w.get("ws1"), ws2=w.get("ws2"), tokens=tokens)


def _step_by_step(cfg, xd, ld, W):
    """The layer through the individual C calls; returns (out, ids, map, offsets)."""
    ids, wts = moe.moe_route_topk(ld, cfg.k, cfg.score, cfg.renormalize, cfg.rsf)
    emap = configs.expert_map(cfg)
    p = moe.moe_permute(ids, cfg.E, cfg.El, None if emap is None else dev(emap), xd)
    h = moe.moe_grouped_gemm1_act(p["x_perm"], p["offsets"], W["w1"], cfg.I)
    y = moe.moe_grouped_gemm2(h, p["offsets"], W["w2"], cfg.H)
    shared = None
    if cfg.shared_I:
        off_s = torch.tensor([0, cfg.T], dtype=torch.int32, device="cuda")
        hs = moe.moe_grouped_gemm1_act(xd, off_s, moe.Weights(W["ws1"].unsqueeze(0)),
                                       cfg.shared_I)
        shared = moe.moe_grouped_gemm2(hs, off_s, moe.Weights(W["ws2"].unsqueeze(0)), cfg.H)
    out = moe.moe_finalize(y, wts, p["map"], 1.0, shared)
    return out, ids, p["map"], p["offsets"]


def test_tiny_every_token():
    cfg = configs.TINY
    x, logits = configs.make_activations(cfg)
    w = configs.make_weights(cfg)
    W = _upload(cfg, w)
    xd, ld = dev_bf16(x), dev(logits)
    ref = _oracle(cfg, x, logits, w)
    out_fused = moe.moe_fused_experts(ld, xd, W["w1"], W["w2"], cfg.k, cfg.score,
                                      cfg.renormalize, cfg.rsf)
    out_steps, ids, pmap, off = _step_by_step(cfg, xd, ld, W)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    assert rel_fro(host_f64(out_fused), ref["out"]) < TOL
    assert np.array_equal(host_bf16_bits(out_fused), host_bf16_bits(out_steps))
    # deferred form, then a separate finalize
    y, ew, m = moe.moe_fused_experts_unfinalized(ld, xd, W["w1"], W["w2"], cfg.k, cfg.score,
                                                 cfg.renormalize, cfg.rsf)
    out_def = moe.moe_finalize(y, ew, m)
    torch.cuda.synchronize()
    assert np.array_equal(m.cpu().numpy(), pmap.cpu().numpy())
    assert rel_fro(host_f64(ew), ref["weights"]) < TOL
    assert rel_fro(host_f64(out_def), ref["out"]) < TOL


def test_tiny_edge_cases():
    cfg = configs.TINY
    x, logits = configs.make_activations(cfg)
    w = configs.make_weights(cfg)
    W = _upload(cfg, w)
    # k = E: every expert on every token
    out = moe.moe_fused_experts(dev(logits), dev_bf16(x), W["w1"], W["w2"], 8, 0, True, 1.0)
    ref = oracle.moe_tokens(x, logits, oracle.Weights(w["w1"]), oracle.Weights(w["w2"]), cfg.I,
                            8, 0, True, 1.0)
    assert rel_fro(host_f64(out), ref["out"]) < TOL
    # T = 0
    e = moe.moe_fused_experts(torch.zeros((0, 8), dtype=torch.float32, device="cuda"),
                              torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda"),
                              W["w1"], W["w2"], 2)
    assert e.shape == (0, 128)
    # a map with no local expert named by any token: output exactly zero
    emap = np.full(8, -1, dtype=np.int32)
    emap[0] = 0
    lg = logits.copy()
    lg[:, 0] = -1e9  # nobody picks expert 0
    w1l = moe.Weights(W["w1"].data[:1].contiguous())
    w2l = moe.Weights(W["w2"].data[:1].contiguous())
    z = moe.moe_fused_experts(dev(lg), dev_bf16(x), w1l, w2l, 2, 0, True, 1.0,
                              expert_map=dev(emap))
    assert torch.all(z == 0)


def _full_size(cfg, n_sample, seed, tol=TOL):
    x, logits = configs.make_activations(cfg)
    w = configs.make_weights(cfg)
    W = _upload(cfg, w)
    xd, ld = dev_bf16(x), dev(logits)
    out_steps, ids, pmap, off = _step_by_step(cfg, xd, ld, W)
    kw = {}
    if cfg.shared_I:
        kw = dict(ws1=W["ws1"], ws2=W["ws2"])
    out1 = moe.moe_fused_experts(ld, xd, W["w1"], W["w2"], cfg.k, cfg.score, cfg.renormalize,
                                 cfg.rsf, **kw)
    out2 = moe.moe_fused_experts(ld, xd, W["w1"], W["w2"], cfg.k, cfg.score, cfg.renormalize,
                                 cfg.rsf, **kw)
    torch.cuda.synchronize()
    ref_ids, _ = oracle.route(logits, cfg.k, cfg.score, cfg.renormalize, cfg.rsf)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    ref_map, ref_off, _ = oracle.permute(ref_ids, cfg.E, cfg.El, configs.expert_map(cfg))
    assert np.array_equal(pmap.cpu().numpy(), ref_map)
    assert np.array_equal(off.cpu().numpy(), ref_off)
    a, b, c = host_bf16_bits(out1), host_bf16_bits(out2), host_bf16_bits(out_steps)
    assert np.array_equal(a, b), "two runs differ"
    assert np.array_equal(a, c), "fused entry point differs from the individual calls"
    toks = sample_tokens(cfg.T, n_sample, seed)
    ref = _oracle(cfg, x, logits, w, tokens=toks)
    got = host_f64(out1)[toks]
    assert np.all(np.isfinite(got))
    assert rel_fro(got, ref["out"]) < tol


def test_mixtral_prefill_full_size():
    _full_size(configs.MIXTRAL, 32, 2)


def test_deepseek_routed_shared_full_size():
    _full_size(configs.DEEPSEEK, 24, 3)


# MXFP4 weights: bar 3e-2 (the weights are exact in both; the GPU rounds h, Y
# and out to bf16 like the bf16 path, so the measured gap is the same ~3e-3).
MXFP4_TOL = 3e-2


def test_deepseek_mxfp4_full_size():
    _full_size(configs.DEEPSEEK_MXFP4, 24, 5, tol=MXFP4_TOL)


def test_tiny_mxfp4_deferred_and_fused():
    cfg = configs.MoeConfig("tiny_mxfp4", T=40, H=256, I=192, E=8, k=2, score=configs.SOFTMAX,
                            renormalize=True, rsf=1.0, seed=6, mxfp4=True)
    x, logits = configs.make_activations(cfg)
    w = configs.make_weights(cfg)
    W = _upload(cfg, w)
    ref = _oracle(cfg, x, logits, w)
    out = moe.moe_fused_experts(dev(logits), dev_bf16(x), W["w1"], W["w2"], cfg.k)
    y, ew, m = moe.moe_fused_experts_unfinalized(dev(logits), dev_bf16(x), W["w1"], W["w2"], cfg.k)
    out2 = moe.moe_finalize(y, ew, m)
    torch.cuda.synchronize()
    assert rel_fro(host_f64(out), ref["out"]) < MXFP4_TOL
    assert rel_fro(host_f64(out2), ref["out"]) < MXFP4_TOL


@pytest.mark.parametrize("T", configs.EP_DECODE_BATCHES)
def test_ep_rank_decode_deferred(T):
    base = configs.EP_DECODE
    w = configs.make_weights(base)
    W = _upload(base, w)
    emap = dev(configs.expert_map(base))
    for d in range(3):  # a few of the routing draws
        cfg = base.with_T(T)
        x, logits = configs.make_activations(cfg, seed=configs.EP_DECODE_DRAW_SEED0 + d)
        R_pad = moe.moe_permuted_rows(T, cfg.k)
        y, ew, m = moe.moe_fused_experts_unfinalized(
            dev(logits), dev_bf16(x), W["w1"], W["w2"], cfg.k, cfg.score, cfg.renormalize,
            cfg.rsf, expert_map=emap, R_pad=R_pad)
        out = moe.moe_finalize(y, ew, m)
        torch.cuda.synchronize()
        ref = _oracle(cfg, x, logits, w)
        ref_map, ref_off, _ = oracle.permute(ref["ids"], cfg.E, cfg.El,
                                             configs.expert_map(cfg))
        mm = m.cpu().numpy()
        assert np.array_equal(mm, ref_map)
        assert y.shape == (R_pad, cfg.H)
        assert rel_fro(host_f64(ew), ref["weights"]) < TOL
        yy = host_f64(y)
        sel = mm >= 0
        if sel.any():
            assert rel_fro(yy[mm[sel]], ref["y_routes"][sel]) < TOL
        assert rel_fro(host_f64(out), ref["out"]) < TOL


@pytest.mark.parametrize("T", [1, 7, 128, 129])
def test_decode_rows_gathered_by_gemm1(T):
    """The fused call lets GEMM1 read its rows from x through the inverse map
    (no gather kernel): bit-identical to the individual calls (which gather
    first) and equal to the oracle, at decode and wider batches, with a
    scattered expert map; the first batch has one token whose routes are all
    non-local."""
    cfg = configs.MoeConfig("gath", T=T, H=1024, I=512, E=64, k=8, score=configs.SIGMOID,
                            renormalize=True, rsf=2.5, seed=70 + T, E_local=16)
    emap = np.full(cfg.E, -1, dtype=np.int32)
    local = np.arange(3, 64, 4)[:16]          # scattered global ids 3, 7, 11, ...
    emap[local] = np.arange(16, dtype=np.int32)
    x, logits = configs.make_activations(cfg)
    if T == 1:
        logits[0, local] = -1e9               # no local route at all
    w = configs.make_weights(cfg)
    W1, W2 = moe.Weights(dev_bf16(w["w1"])), moe.Weights(dev_bf16(w["w2"]))
    xd, ld, ed = dev_bf16(x), dev(logits), dev(emap)
    out = moe.moe_fused_experts(ld, xd, W1, W2, cfg.k, cfg.score, True, cfg.rsf, expert_map=ed)
    ids, wts = moe.moe_route_topk(ld, cfg.k, cfg.score, True, cfg.rsf)
    p = moe.moe_permute(ids, cfg.E, 16, ed, xd)
    h = moe.moe_grouped_gemm1_act(p["x_perm"], p["offsets"], W1, cfg.I)
    y = moe.moe_grouped_gemm2(h, p["offsets"], W2, cfg.H)
    out_steps = moe.moe_finalize(y, wts, p["map"])
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(out), host_bf16_bits(out_steps))
    ref = oracle.moe_tokens(x, logits, oracle.Weights(w["w1"]), oracle.Weights(w["w2"]), cfg.I,
                            cfg.k, cfg.score, True, cfg.rsf, expert_map=emap)
    assert rel_fro(host_f64(out), ref["out"]) < TOL
    if T == 1:
        assert torch.all(out == 0)


@pytest.mark.parametrize("mxfp4", [False, True], ids=["bf16", "mxfp4"])
@pytest.mark.parametrize("T,split", [(3, True), (40, True), (40, False), (300, False)])
def test_gemm1_gathered_equals_gather_then_gemm1(T, split, mxfp4):
    """moe_grouped_gemm1_act_gathered(x, inv) is moe_permute's gather followed by
    moe_grouped_gemm1_act, bit for bit (decode tiles with and without split
    reductions, and a wider batch), NaN in the unread padding rows of h's input."""
    E, E_l, k, H, I = 32, 8, 4, 512, 256
    x = synth.normal_bf16(80 + T, 0, (T, H))
    logits = synth.normal_f32(80 + T, 1, (T, E))
    emap = np.full(E, -1, dtype=np.int32)
    emap[8:16] = np.arange(8, dtype=np.int32)
    w1 = synth.normal_bf16(80 + T, 2, (E_l, 2 * I, H), std=1 / np.sqrt(H))
    if mxfp4:
        q, sc = synth.mxfp4_quantize(w1)
        W1 = moe.Weights(dev(q), dev(sc))
    else:
        W1 = moe.Weights(dev_bf16(w1))
    xd = dev_bf16(x)
    ids, _ = moe.moe_route_topk(dev(logits), k, moe.SIGMOID)
    p = moe.moe_permute(ids, E, E_l, dev(emap), xd)
    R_l = int(p["offsets"][-1].item())
    p["x_perm"][R_l:] = float("nan")
    h_ref = moe.moe_grouped_gemm1_act(p["x_perm"], p["offsets"], W1, I, split=split)
    h = moe.moe_grouped_gemm1_act_gathered(xd, p["inv"], k, p["offsets"], W1, I, split=split)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(h)[:R_l], host_bf16_bits(h_ref)[:R_l])
    assert R_l > 0
