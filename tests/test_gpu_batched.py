"""GPU parity of the batched experts format (modular_kernel.py:
FusedMoEActivationFormat.BatchedExperts, (local experts, max tokens per
expert, hidden) with expert_num_tokens) against the oracle.

- moe_permute_batched: map and counts bit-exact against oracle.permute_batched,
  with and without an expert map, with routes dropped past a capacity; the
  gathered rows bit-exact (plain and weight-scaled);
- the two batched GEMMs against oracle.hidden_rows / out_rows on every kept
  row, for decode-like, wide, split and large blocks; NaN planted in the
  unused rows of every block never reaches the outputs, and unused output
  rows stay untouched;
- whole layers in the batched format: bit-identical to the standard layout
  when no reduction is split (same tiles, same reduction order), against the
  oracle, in the deferred form at the expert-parallel decode shape, and with
  dropped routes against the oracle's per-route outputs summed over the kept
  routes.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_scan_amd as moe
import oracle
import synth
from synth import configs

from gpu_util import dev, dev_bf16, host_bf16_bits, host_f64, need_gpu, rel_fro, sample_tokens

pytestmark = pytest.mark.gpu

TOL = 1e-2
NAN_BITS = 0x7FC0


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _route(T, E, k, seed, hot=None):
    logits = synth.normal_f32(seed, 1, (T, E))
    if hot is not None:
        logits[:, hot] += 3.0
    ids, wts = moe.moe_route_topk(dev(logits), k, configs.SOFTMAX, True, 1.0)
    return logits, ids, wts


@pytest.mark.parametrize("T,E,E_l,k,M,use_map", [
    (40, 8, 8, 2, 40, False),     # capacity T: nothing drops
    (64, 8, 8, 4, 20, False),     # expert 3 overflows its 20 slots
    (33, 16, 4, 3, 8, True),      # expert-parallel map, 4 local experts
    (1, 8, 8, 2, 1, False),       # one token
    # several permute workgroups (one per 1024 routes), with drops
    (1500, 8, 8, 2, 300, False),  # 3000 routes, expert 3 overflows
    (1200, 16, 4, 3, 600, True),  # 3600 routes, expert-parallel map
])
def test_permute_batched_bit_exact(T, E, E_l, k, M, use_map):
    H = 136
    logits, ids, wts = _route(T, E, k, seed=T + M, hot=3 if M < T else None)
    emap = None
    if use_map:
        emap = np.full(E, -1, dtype=np.int32)
        emap[[2, 5, 9, 14]] = np.arange(4, dtype=np.int32)
    x = synth.normal_bf16(T + M, 0, (T, H))
    xb = torch.full((E_l, M, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    p = moe.moe_permute_batched(ids, E, M, E_l, None if emap is None else dev(emap),
                                dev_bf16(x), x_batched=xb)
    xs = torch.full((E_l, M, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ps = moe.moe_permute_batched(ids, E, M, E_l, None if emap is None else dev(emap),
                                 dev_bf16(x), x_batched=xs, x_weights=wts)
    torch.cuda.synchronize()
    ref_map, ref_cnt = oracle.permute_batched(ids.cpu().numpy(), E, E_l, M, emap)
    m = p["map"].cpu().numpy()
    assert np.array_equal(m, ref_map)
    assert np.array_equal(p["expert_num_tokens"].cpu().numpy(), ref_cnt)
    assert np.array_equal(ps["map"].cpu().numpy(), ref_map)
    if M < T and not use_map:
        assert ref_cnt.max() > M  # the overflow case really drops routes
    got = host_bf16_bits(xb).reshape(E_l * M, H)
    got_s = host_bf16_bits(xs).reshape(E_l * M, H)
    w32 = wts.cpu().numpy()
    xf = synth.bf16_bits_to_f32(x)
    used = np.zeros(E_l * M, dtype=bool)
    for t in range(T):
        for j in range(k):
            r = m[t, j]
            if r < 0:
                continue
            used[r] = True
            assert np.array_equal(got[r], x[t])
            u = (np.float32(w32[t, j]) * xf[t]).astype(np.float32).view(np.uint32).astype(np.uint64)
            assert np.array_equal(got_s[r], ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16))
    assert np.all(got[~used] == NAN_BITS)  # slots past each count are not written


GEMM_CASES = [
    # name, counts per local expert, max_tokens, H, I
    ("decode_blocks", [0, 1, 0, 3, 2, 0, 0, 1] * 4, 8, 512, 256),
    ("wide_blocks", [20, 0, 100, 64, 31, 97], 128, 256, 192),
    ("split_blocks", [1, 0, 2, 1, 0, 3], 16, 1024, 512),
    ("large_blocks", [700, 613], 768, 512, 384),
]


def _segments(counts, M):
    """(kept row indices in the batched layout, expert of each kept row)."""
    rows, eor = [], []
    for e, c in enumerate(counts):
        rows.extend(range(e * M, e * M + min(c, M)))
        eor.extend([e] * min(c, M))
    return np.array(rows, dtype=np.int64), np.array(eor, dtype=np.int32)


@pytest.mark.parametrize("case", GEMM_CASES, ids=[c[0] for c in GEMM_CASES])
def test_batched_gemms(case):
    name, counts, M, H, I = case
    E_l = len(counts)
    seed = sum(counts) + 61
    rows, eor = _segments(counts, M)
    a = synth.normal_bf16(seed, 0, (E_l * M, H))
    hb = synth.normal_bf16(seed, 7, (E_l * M, I))
    unused = np.ones(E_l * M, dtype=bool)
    unused[rows] = False
    a[unused] = NAN_BITS   # never read
    hb[unused] = NAN_BITS
    w1 = synth.normal_bf16(seed, 2, (E_l, 2 * I, H), std=1 / np.sqrt(H))
    w2 = synth.normal_bf16(seed, 3, (E_l, H, I), std=1 / np.sqrt(I))
    cnt = dev(np.array(counts, dtype=np.int32))
    h = torch.full((E_l, M, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = torch.full((E_l, M, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm1_act_batched(dev_bf16(a).view(E_l, M, H), cnt, moe.Weights(dev_bf16(w1)),
                                      I, h_batched=h, max_rows=int(sum(counts)))
    moe.moe_grouped_gemm2_batched(dev_bf16(hb).view(E_l, M, I), cnt, moe.Weights(dev_bf16(w2)), H,
                                  y_batched=y)
    torch.cuda.synchronize()
    ref_h = oracle.hidden_rows(a[rows], oracle.Weights(w1), eor, I)
    ref_y = oracle.out_rows(hb[rows], oracle.Weights(w2), eor, H)
    got_h = host_f64(h).reshape(E_l * M, I)
    got_y = host_f64(y).reshape(E_l * M, H)
    assert rel_fro(got_h[rows], ref_h) < TOL
    assert rel_fro(got_y[rows], ref_y) < TOL
    assert np.all(host_bf16_bits(h).reshape(E_l * M, I)[unused] == NAN_BITS)
    assert np.all(host_bf16_bits(y).reshape(E_l * M, H)[unused] == NAN_BITS)


def _small(name, T, H, I, E, k, seed, shared_I=0):
    return configs.MoeConfig(name, T=T, H=H, I=I, E=E, k=k, score=configs.SOFTMAX,
                             renormalize=True, rsf=1.0, seed=seed, shared_I=shared_I)


def test_batched_layer_equals_standard_layout():
    cfg = _small("b", T=300, H=256, I=320, E=8, k=2, seed=62, shared_I=128)
    x, logits = configs.make_activations(cfg)
    w = configs.make_weights(cfg)
    W1, W2 = moe.Weights(dev_bf16(w["w1"])), moe.Weights(dev_bf16(w["w2"]))
    ws1, ws2 = dev_bf16(w["ws1"]), dev_bf16(w["ws2"])
    xd, ld = dev_bf16(x), dev(logits)
    std = moe.moe_fused_experts(ld, xd, W1, W2, cfg.k, ws1=ws1, ws2=ws2)
    bat = moe.moe_fused_experts(ld, xd, W1, W2, cfg.k, ws1=ws1, ws2=ws2, batched_max_tokens=cfg.T)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(bat), host_bf16_bits(std))
    toks = sample_tokens(cfg.T, 24, 5)
    ref = oracle.moe_tokens(x, logits, oracle.Weights(w["w1"]), oracle.Weights(w["w2"]), cfg.I,
                            cfg.k, cfg.score, True, 1.0, shared_I=cfg.shared_I, ws1=w["ws1"],
                            ws2=w["ws2"], tokens=toks)
    assert rel_fro(host_f64(bat, toks), ref["out"]) < TOL


@pytest.mark.parametrize("T", [1, 64])
def test_batched_deferred_ep_decode(T):
    base = configs.EP_DECODE
    w = configs.make_weights(base)
    W1, W2 = moe.Weights(dev_bf16(w["w1"])), moe.Weights(dev_bf16(w["w2"]))
    emap_np = configs.expert_map(base)
    emap = dev(emap_np)
    cfg = base.with_T(T)
    x, logits = configs.make_activations(cfg, seed=configs.EP_DECODE_DRAW_SEED0 + 2)
    xd, ld = dev_bf16(x), dev(logits)
    args = (ld, xd, W1, W2, cfg.k, cfg.score, cfg.renormalize, cfg.rsf)
    y_s, ew_s, m_s = moe.moe_fused_experts_unfinalized(*args, expert_map=emap)
    y_b, ew_b, m_b = moe.moe_fused_experts_unfinalized(*args, expert_map=emap,
                                                       batched_max_tokens=T)
    out_s = moe.moe_finalize(y_s, ew_s, m_s)
    out_b = moe.moe_finalize(y_b, ew_b, m_b)
    torch.cuda.synchronize()
    assert y_b.shape == (cfg.El * T, cfg.H)
    ids_ref, _ = oracle.route(logits, cfg.k, cfg.score, cfg.renormalize, cfg.rsf)
    ref_map, ref_cnt = oracle.permute_batched(ids_ref, cfg.E, cfg.El, T, emap_np)
    assert np.array_equal(m_b.cpu().numpy(), ref_map)
    assert np.array_equal(host_bf16_bits(ew_b), host_bf16_bits(ew_s))
    # the split reductions may cut the long k-range into other piece counts
    # (the scratch slices span all rows of the layout), so compare to rounding
    assert rel_fro(host_f64(out_b), host_f64(out_s)) < TOL
    ref = oracle.moe_tokens(x, logits, oracle.Weights(w["w1"]), oracle.Weights(w["w2"]), cfg.I,
                            cfg.k, cfg.score, cfg.renormalize, cfg.rsf, expert_map=emap_np)
    assert rel_fro(host_f64(out_b), ref["out"]) < TOL


def test_batched_layer_with_dropped_routes():
    cfg = _small("d", T=96, H=256, I=192, E=8, k=2, seed=63)
    x, logits = configs.make_activations(cfg)
    logits[:, 1] += 2.5   # expert 1 takes most tokens and overflows
    M = 24
    w = configs.make_weights(cfg)
    W1, W2 = moe.Weights(dev_bf16(w["w1"])), moe.Weights(dev_bf16(w["w2"]))
    out = moe.moe_fused_experts(dev(logits), dev_bf16(x), W1, W2, cfg.k, batched_max_tokens=M)
    torch.cuda.synchronize()
    ref = oracle.moe_tokens(x, logits, oracle.Weights(w["w1"]), oracle.Weights(w["w2"]), cfg.I,
                            cfg.k, cfg.score, True, 1.0)
    bmap, cnt = oracle.permute_batched(ref["ids"], cfg.E, cfg.E, M)
    assert cnt.max() > M
    kept = (bmap >= 0)[:, :, None]
    want = np.sum(np.where(kept, ref["weights"][:, :, None] * ref["y_routes"], 0.0), axis=1)
    assert rel_fro(host_f64(out), want) < TOL
    assert rel_fro(want, ref["out"]) > 5 * TOL  # the drops matter
