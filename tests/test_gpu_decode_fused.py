"""GPU parity of moe_route_permute_gemm1_act: router, permute map and GEMM1 in
one call (one kernel for small bf16 decode batches, else the router-permute
and gathered GEMM1 kernels).

Bar: ids, map, offsets and inverse map bit-exact against the oracle; the
hidden rows bit-identical to the separate moe_route_permute +
moe_grouped_gemm1_act_gathered calls (the same per-slice arithmetic) and
within the bf16 bar (relative Frobenius 1e-2) of the oracle's hidden rows;
routing weights within 1e-5 (fp32 against fp64)."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_scan_amd as moe
import oracle
import synth
from synth import configs

from gpu_util import dev, dev_bf16, host_bf16_bits, host_f64, need_gpu, rel_fro, segments_of

pytestmark = pytest.mark.gpu

TOL = 1e-2
W_TOL = 1e-5


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


CASES = [
    # name, T, E, E_l (None: all local, "ep": one rank of 8), k, H, I, score, renorm, rsf, seed
    # one kernel (T <= 8, T * k <= 64, few rows per local expert)
    ("ep_decode_1", 1, 256, "ep", 8, 1024, 512, 1, True, 2.5, 600),
    ("ep_decode_5", 5, 256, "ep", 8, 1024, 512, 1, True, 2.5, 601),
    ("ep_decode_8", 8, 256, "ep", 8, 1024, 512, 1, True, 2.5, 602),
    ("ep_decode_8_short_k", 8, 256, "ep", 8, 768, 256, 1, True, 2.5, 603),
    ("all_local_1024_top32", 2, 1024, None, 32, 512, 256, 1, True, 2.5, 604),
    ("softmax_no_renorm_16_of_64", 8, 64, 16, 4, 512, 256, 0, False, 1.0, 605),
    # past the one-kernel limits: the router-permute and GEMM1 kernels
    ("two_launches_T9", 9, 256, "ep", 8, 1024, 512, 1, True, 2.5, 606),
    ("two_launches_many_rows", 8, 8, None, 2, 512, 256, 0, True, 1.0, 607),
]


def _emap(E, El, seed):
    if El is None:
        return None, E
    if El == "ep":
        cfg = configs.EP_DECODE
        return configs.expert_map(cfg), cfg.El
    rng = np.random.default_rng(seed)
    m = np.full(E, -1, dtype=np.int32)
    m[rng.choice(E, El, replace=False)] = rng.permutation(El).astype(np.int32)
    return m, El


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_route_permute_gemm1(case):
    name, T, E, El, k, H, I, score, renorm, rsf, seed = case
    emap, E_l = _emap(E, El, seed)
    logits = synth.normal_f32(seed, synth.TID_LOGITS, (T, E))
    x = synth.normal_bf16(seed, synth.TID_X, (T, H))
    w1 = synth.normal_bf16(seed, synth.TID_W1, (E_l, 2 * I, H), std=1 / np.sqrt(H))
    W1 = moe.Weights(dev_bf16(w1))
    R_pad = configs.permuted_rows(T, k)
    ld, xd = dev(logits), dev_bf16(x)
    ed = None if emap is None else dev(emap)
    h0 = torch.full((R_pad, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    r = moe.moe_route_permute_gemm1_act(ld, xd, k, W1, I, score, renorm, rsf, ed, R_pad, h=h0)
    # the separate calls
    p = moe.moe_route_permute(ld, k, score, renorm, rsf, E_l, ed, R_pad)
    h1 = moe.moe_grouped_gemm1_act_gathered(xd, p["inv"], k, p["offsets"], W1, I)
    torch.cuda.synchronize()
    ref_ids, ref_w = oracle.route(logits, k, score, renorm, rsf)
    assert np.array_equal(r["topk_ids"].cpu().numpy(), ref_ids)
    assert rel_fro(r["topk_weights"].cpu().numpy(), ref_w) < W_TOL
    ref_map, ref_off, _ = oracle.permute(ref_ids, E, E_l, emap)
    assert np.array_equal(r["map"].cpu().numpy(), ref_map)
    assert np.array_equal(r["offsets"].cpu().numpy(), ref_off)
    want_inv = np.full(R_pad, -1, dtype=np.int64)
    flat = ref_map.reshape(-1)
    want_inv[flat[flat >= 0]] = np.nonzero(flat >= 0)[0]
    assert np.array_equal(r["inv"].cpu().numpy(), want_inv)
    R_l = int(ref_off[-1])
    got = host_bf16_bits(r["h"])
    assert np.array_equal(got[:R_l], host_bf16_bits(h1)[:R_l])
    # rows past the local routes are not written
    assert np.all(got[R_l:] == 0x7FC0)
    if R_l:
        ref_h = oracle.hidden_rows(x[want_inv[:R_l] // k], oracle.Weights(w1),
                                   segments_of(ref_off, R_l), I)
        assert rel_fro(host_f64(r["h"], slice(None, R_l)), ref_h) < TOL


def test_route_permute_gemm1_gelu_clamp():
    """The activation options reach the fused kernel's epilogue."""
    T, E, k, H, I = 4, 256, 8, 512, 256
    emap, E_l = _emap(E, "ep", 0)
    logits = synth.normal_f32(610, synth.TID_LOGITS, (T, E))
    x = synth.normal_bf16(610, synth.TID_X, (T, H))
    w1 = synth.normal_bf16(610, synth.TID_W1, (E_l, 2 * I, H), std=1 / np.sqrt(H))
    W1 = moe.Weights(dev_bf16(w1))
    ld, xd, ed = dev(logits), dev_bf16(x), dev(emap)
    for act, clamp in [(moe.ACT_GELU, None), (moe.ACT_SILU, 0.5)]:
        r = moe.moe_route_permute_gemm1_act(ld, xd, k, W1, I, 1, True, 2.5, ed,
                                            activation=act, activation_clamp=clamp)
        p = moe.moe_route_permute(ld, k, 1, True, 2.5, E_l, ed)
        h1 = moe.moe_grouped_gemm1_act_gathered(xd, p["inv"], k, p["offsets"], W1, I,
                                                activation=act, activation_clamp=clamp)
        torch.cuda.synchronize()
        R_l = int(p["offsets"][-1].item())
        assert np.array_equal(host_bf16_bits(r["h"])[:R_l], host_bf16_bits(h1)[:R_l])


def test_route_permute_gemm1_empty():
    W1 = moe.Weights(torch.zeros((4, 512, 256), dtype=torch.bfloat16, device="cuda"))
    r = moe.moe_route_permute_gemm1_act(torch.zeros((0, 4), dtype=torch.float32, device="cuda"),
                                        torch.zeros((0, 256), dtype=torch.bfloat16,
                                                    device="cuda"), 2, W1, 256)
    torch.cuda.synchronize()
    assert np.all(r["offsets"].cpu().numpy() == 0)
