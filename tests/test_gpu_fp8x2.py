"""GPU parity of the two-term FP8 activations with MXFP4 weights (bf16
activations carried to the FP8 x e2m1 matrix cores as scale * (q1 + q2 / 16))
against the oracle.

- moe_quantize_fp8x2: both terms' codes and the scales bit-exact against the
  oracle's float32 two-term quantizer (zero rows, row weights, wide rows),
  in the interleaved row layout (per 64 k, 64 codes of q1 then 64 of q2);
- both two-term GEMMs on every tile shape and on the split path, against the
  oracle on the same codes (bar 1e-2: only fp32 accumulation order and the
  bf16 output rounding separate the two sides);
- whole layers (fused, deferred, chunked, the EP decode shape) against the
  oracle's two-term mode (1e-2) and against the plain bf16-activation oracle
  (3e-2, the MXFP4 bar), and the full-size DeepSeek-V3 MXFP4 workload on
  sampled tokens, twice bit-identically.
"""
import gc

import numpy as np
import pytest
import torch

import mixture_experts_layer_scan_amd as moe
import oracle
import synth
from synth import configs

from gpu_util import (covering_tokens, dev, dev_bf16, host_bf16_bits, host_f64, need_gpu,
                      per_row_rel, rel_fro, sample_tokens, segments_of,
                      expert_sample_rows)

pytestmark = pytest.mark.gpu

TOL_SAME = 1e-2   # against the oracle on the same two-term codes
TOL_MXFP4 = 3e-2  # against the bf16-activation oracle (the MXFP4 bar)


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _split_terms(q: np.ndarray):
    """[rows, 2H] interleaved per 64 k -> (q1 [rows, H], q2 [rows, H])."""
    rows, H2 = q.shape
    b = q.reshape(rows, H2 // 128, 2, 64)
    return (np.ascontiguousarray(b[:, :, 0, :].reshape(rows, H2 // 2)),
            np.ascontiguousarray(b[:, :, 1, :].reshape(rows, H2 // 2)))


def _join_terms(q1: np.ndarray, q2: np.ndarray) -> np.ndarray:
    rows, H = q1.shape
    return np.ascontiguousarray(np.stack([q1.reshape(rows, H // 64, 64),
                                          q2.reshape(rows, H // 64, 64)], axis=2)
                                .reshape(rows, 2 * H))


def _rne_bf16(xf: np.ndarray) -> np.ndarray:
    u = xf.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("rows,H,mode", [(37, 256, "plain"), (5, 7168, "plain"),
                                         (9, 2048, "weights"), (3, 64, "plain")])
def test_quantize_x2_bit_exact(rows, H, mode):
    x = synth.normal_bf16(rows + H, 0, (rows, H), std=3.0)
    x[min(2, rows - 1)] = 0
    x[0, :6] = [0x3C00, 0xBC00, 0x0001, 0x8001, 0x4380, 0xC3E0]  # odd values
    rw = synth.normal_f32(rows, 3, (rows,)) if mode == "weights" else None
    q, sc = moe.moe_quantize_fp8x2(dev_bf16(x), None if rw is None else dev(rw))
    torch.cuda.synchronize()
    x_in = x if rw is None else _rne_bf16(synth.bf16_bits_to_f32(x) * rw[:, None])
    r1, r2, rs = oracle.quantize_fp8x2_rows(x_in)
    g1, g2 = _split_terms(q.cpu().numpy())
    assert np.array_equal(g1, r1)
    assert np.array_equal(g2, r2)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def test_quantize_x2_row_count_and_permute():
    """Only rows below *row_count are written; moe_permute_fp8 moves rows of
    2H bytes with their scales."""
    T, k, E, H = 40, 2, 8, 256
    x = synth.normal_bf16(97, 0, (T, H))
    q = torch.full((T, 2 * H), 0x7F, dtype=torch.uint8, device="cuda")
    sc = torch.full((T,), -1.0, dtype=torch.float32, device="cuda")
    moe.moe_quantize_fp8x2(dev_bf16(x), None, q, sc, row_count=dev(np.array([25], np.int32)))
    logits = synth.normal_f32(97, 1, (T, E))
    ids, _ = moe.moe_route_topk(dev(logits), k)
    qa, sa = moe.moe_quantize_fp8x2(dev_bf16(x))
    p = moe.moe_permute_fp8(ids, E, qa, sa)
    torch.cuda.synchronize()
    qn = q.cpu().numpy()
    r1, r2, rs = oracle.quantize_fp8x2_rows(x)
    g1, g2 = _split_terms(qn[:25])
    assert np.array_equal(g1, r1[:25]) and np.array_equal(g2, r2[:25])
    assert np.all(qn[25:] == 0x7F) and np.all(sc.cpu().numpy()[25:] == -1.0)
    m = p["map"].cpu().numpy()
    gq, gs = p["xq_perm"].cpu().numpy(), p["xq_perm_scales"].cpu().numpy()
    full = _join_terms(r1, r2)
    for t in range(T):
        for j in range(k):
            assert np.array_equal(gq[m[t, j]], full[t]) and gs[m[t, j]] == rs[t]


X2_CASES = [
    # name, counts per local expert, H, I (multiples of 256: MXFP4 weight stages)
    ("thin_tiles", [0, 1, 5, 33, 2, 0, 17, 40], 256, 256),
    ("wide_tiles", [70, 0, 130, 55], 512, 256),
    ("wide_ragged_fragments", [0, 3, 129, 31, 64, 97], 256, 256),
    ("mid_tiles", [300, 1, 420], 256, 512),
    ("big_tiles", [700, 613], 512, 256),
    ("split_decode", [1, 0, 2, 1, 0, 3], 1024, 512),
    ("split_wide", [20, 30, 0, 16], 1024, 512),
]


@pytest.mark.parametrize("split", [True, False], ids=["split_ok", "no_split"])
@pytest.mark.parametrize("case", X2_CASES, ids=[c[0] for c in X2_CASES])
def test_x2_gemms(case, split):
    name, counts, H, I = case
    E_l = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R_l = int(offsets[-1])
    R_pad = ((R_l + 127) // 128) * 128
    seed = sum(counts) + 98
    a1, a2, asc = oracle.quantize_fp8x2_rows(synth.normal_bf16(seed, 0, (R_pad, H)))
    h1, h2, hsc = oracle.quantize_fp8x2_rows(synth.normal_bf16(seed, 7, (R_pad, I)))
    for t in (a1, a2, h1, h2):
        t[R_l:] = 0x7F   # E4M3 NaN in rows the kernels must not read
    q1, s1 = synth.mxfp4_quantize(synth.normal_bf16(seed, 2, (E_l, 2 * I, H), std=1 / np.sqrt(H)))
    q2, s2 = synth.mxfp4_quantize(synth.normal_bf16(seed, 3, (E_l, H, I), std=1 / np.sqrt(I)))
    off = dev(offsets)
    h = moe.moe_grouped_gemm1_act_fp8x2(dev(_join_terms(a1, a2)), dev(asc), off,
                                        moe.Weights(dev(q1), dev(s1)), I, split=split)
    y = moe.moe_grouped_gemm2_fp8x2(dev(_join_terms(h1, h2)), dev(hsc), off,
                                    moe.Weights(dev(q2), dev(s2)), H, split=split)
    torch.cuda.synchronize()
    eor = segments_of(offsets, R_l)
    ref_h = oracle.hidden_rows_fp8x2(a1[:R_l], a2[:R_l], asc[:R_l], oracle.Weights(q1, s1), eor, I)
    ref_y = oracle.out_rows_fp8x2(h1[:R_l], h2[:R_l], hsc[:R_l], oracle.Weights(q2, s2), eor, H)
    assert rel_fro(host_f64(h, slice(None, R_l)), ref_h) < TOL_SAME
    assert rel_fro(host_f64(y, slice(None, R_l)), ref_y) < TOL_SAME


def _upload(w):
    return (moe.Weights(dev(w["w1_q"]), dev(w["w1_s"])),
            moe.Weights(dev(w["w2_q"]), dev(w["w2_s"])))


def _ref(cfg, x, logits, w, fp8="x2", **kw):
    return oracle.moe_tokens(x, logits, oracle.Weights(w["w1_q"], w["w1_s"]),
                             oracle.Weights(w["w2_q"], w["w2_s"]), cfg.I, cfg.k, cfg.score,
                             cfg.renormalize, cfg.rsf, expert_map=configs.expert_map(cfg),
                             fp8=fp8, **kw)


@pytest.mark.parametrize("chunk", [0, 96])
def test_x2_layer_fused_and_deferred(chunk):
    cfg = configs.MoeConfig("x2", T=300, H=512, I=256, E=16, k=4, score=configs.SIGMOID,
                            renormalize=True, rsf=2.5, seed=99, mxfp4=True, fp8x2=True)
    x, logits = configs.make_activations(cfg)
    w = configs.make_weights(cfg)
    W1, W2 = _upload(w)
    args = (dev(logits), dev_bf16(x), W1, W2, cfg.k, cfg.score, cfg.renormalize, cfg.rsf)
    out = moe.moe_fused_experts(*args, fp8="x2", chunk_tokens=chunk)
    y, ew, m = moe.moe_fused_experts_unfinalized(*args, fp8="x2")
    fin = moe.moe_finalize(y, ew, m)
    torch.cuda.synchronize()
    ref = _ref(cfg, x, logits, w)
    plain = _ref(cfg, x, logits, w, fp8=False)
    assert rel_fro(host_f64(out), ref["out"]) < TOL_SAME
    assert rel_fro(host_f64(fin), ref["out"]) < TOL_SAME
    assert rel_fro(host_f64(out), plain["out"]) < TOL_MXFP4
    mm = m.cpu().numpy()
    assert rel_fro(host_f64(y, mm.reshape(-1)), ref["y_routes"].reshape(-1, cfg.H)) < TOL_SAME


@pytest.mark.parametrize("T", [1, 8, 64])
def test_x2_ep_decode_deferred(T):
    base = configs.EP_DECODE
    cfg = configs.MoeConfig("ep_x2", T=T, H=base.H, I=base.I, E=base.E, k=base.k,
                            score=base.score, renormalize=True, rsf=base.rsf, seed=base.seed,
                            E_local=base.E_local, local_first=base.local_first, mxfp4=True,
                            fp8x2=True)
    w = configs.make_weights(cfg)
    W1, W2 = _upload(w)
    emap = configs.expert_map(cfg)
    x, logits = configs.make_activations(cfg, seed=configs.EP_DECODE_DRAW_SEED0 + 2)
    y, ew, m = moe.moe_fused_experts_unfinalized(dev(logits), dev_bf16(x), W1, W2, cfg.k,
                                                 cfg.score, True, cfg.rsf,
                                                 expert_map=dev(emap), fp8="x2")
    out = moe.moe_finalize(y, ew, m)
    torch.cuda.synchronize()
    ref = _ref(cfg, x, logits, w)
    assert rel_fro(host_f64(out), ref["out"]) < TOL_SAME


def test_x2_rejects_other_weights_and_static_scales():
    cfg = configs.MoeConfig("x2r", T=8, H=256, I=256, E=4, k=2, score=configs.SOFTMAX,
                            renormalize=True, rsf=1.0, seed=3)
    x, logits = configs.make_activations(cfg)
    w = configs.make_weights(cfg)
    W1, W2 = moe.Weights(dev_bf16(w["w1"])), moe.Weights(dev_bf16(w["w2"]))
    with pytest.raises(RuntimeError):
        moe.moe_fused_experts(dev(logits), dev_bf16(x), W1, W2, 2, fp8="x2")


def test_x2_full_size_deepseek_mxfp4():
    cfg = configs.DEEPSEEK_MXFP4
    x, logits = configs.make_activations(cfg)
    w = configs.make_weights(cfg)
    W1, W2 = _upload(w)
    xd, ld = dev_bf16(x), dev(logits)
    out = moe.moe_fused_experts(ld, xd, W1, W2, cfg.k, cfg.score, cfg.renormalize, cfg.rsf,
                                fp8="x2")
    out2 = moe.moe_fused_experts(ld, xd, W1, W2, cfg.k, cfg.score, cfg.renormalize, cfg.rsf,
                                 fp8="x2")
    # the stages one by one, as the benchmark times them
    k, H, I, E_l = cfg.k, cfg.H, cfg.I, cfg.El
    ids_d, wts_d = moe.moe_route_topk(ld, k, cfg.score, cfg.renormalize, cfg.rsf)
    xq, xs = moe.moe_quantize_fp8x2(xd)
    p = moe.moe_permute_fp8(ids_d, cfg.E, xq, xs)
    h = moe.moe_grouped_gemm1_act_fp8x2(p["xq_perm"], p["xq_perm_scales"], p["offsets"], W1, I)
    hq, hs = moe.moe_quantize_fp8x2(h, None, row_count=p["offsets"][E_l:])
    y = moe.moe_grouped_gemm2_fp8x2(hq, hs, p["offsets"], W2, H)
    out_s = moe.moe_finalize(y, wts_d, p["map"])
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(out), host_bf16_bits(out2))
    assert np.array_equal(host_bf16_bits(out), host_bf16_bits(out_s))
    # h and Y rows of every expert against the oracle's row functions on the
    # kernels' own codes (the codes themselves are pinned bit for bit above)
    off = p["offsets"].cpu().numpy()
    R_l = int(off[-1])
    rows = expert_sample_rows(off, 2, 11)
    eor = segments_of(off, R_l)[rows]
    W1o, W2o = oracle.Weights(w["w1_q"], w["w1_s"]), oracle.Weights(w["w2_q"], w["w2_s"])
    a1, a2 = _split_terms(p["xq_perm"].cpu().numpy()[rows])
    ref_h = oracle.hidden_rows_fp8x2(a1, a2, p["xq_perm_scales"].cpu().numpy()[rows], W1o, eor, I)
    e_h = per_row_rel(host_f64(h, rows), ref_h)
    b1, b2 = _split_terms(hq.cpu().numpy()[rows])
    ref_y = oracle.out_rows_fp8x2(b1, b2, hs.cpu().numpy()[rows], W2o, eor, H)
    e_y = per_row_rel(host_f64(y, rows), ref_y)
    print(f"\n{cfg.name}: {len(rows)} h rows of {len(np.unique(eor))} experts, max {e_h.max():.2e}; "
          f"Y rows max {e_y.max():.2e}")
    assert len(np.unique(eor)) == E_l
    assert e_h.max() < TOL_SAME and e_y.max() < TOL_SAME
    # tokens whose routes reach every expert, per token and pooled, against the
    # oracle on the same two-term codes and against the bf16-activation layer
    ids, _ = oracle.route(logits, cfg.k, cfg.score, cfg.renormalize, cfg.rsf)
    toks = covering_tokens(ids, 256, 10)
    got = host_f64(out, toks)
    assert np.all(np.isfinite(got))
    same = _ref(cfg, x, logits, w, tokens=toks)["out"]
    plain = _ref(cfg, x, logits, w, fp8=False, tokens=toks)["out"]
    e_same, e_plain = per_row_rel(got, same), per_row_rel(got, plain)
    print(f"\n{cfg.name}: {len(toks)} tokens reaching {len(np.unique(ids[toks]))} experts; "
          f"same codes per-token max {e_same.max():.2e} pooled {rel_fro(got, same):.2e}; "
          f"bf16 activations per-token max {e_plain.max():.2e} pooled {rel_fro(got, plain):.2e}")
    assert len(np.unique(ids[toks])) == cfg.E
    assert e_same.max() < TOL_SAME and rel_fro(got, same) < TOL_SAME
    assert e_plain.max() < TOL_MXFP4 and rel_fro(got, plain) < TOL_MXFP4
