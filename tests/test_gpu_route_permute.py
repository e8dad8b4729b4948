"""GPU parity of the router and the permute step against the oracle.

Bar: expert ids, permute map, offsets and inverse map bit-exact; gathered rows
bit-exact (pure byte movement); routing weights (fp32 on the GPU, fp64 in the
oracle) within a relative Frobenius error of 1e-5 (fp32 exp / division
rounding is ~1e-7; the layer-level bar of 1e-2 is far looser)."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_scan_amd as moe
import oracle
import synth
from synth import configs

from gpu_util import dev, dev_bf16, host_bf16_bits, need_gpu, rel_fro

pytestmark = pytest.mark.gpu

W_TOL = 1e-5


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


ROUTE_CASES = [
    # name, T, E, k, score, renormalize, rsf, seed, zipf
    ("tiny_softmax_top2", 16, 8, 2, 0, True, 1.0, 1, 0.0),
    ("mixtral_zipf_4096x8_top2", 4096, 8, 2, 0, True, 1.0, 2, 1.1),
    ("deepseek_2048x256_top8_sigmoid", 2048, 256, 8, 1, True, 2.5, 3, 0.0),
    ("decode_1x256_top8", 1, 256, 8, 1, True, 2.5, 400, 0.0),
    ("ragged_13x100_top5", 13, 100, 5, 0, True, 1.0, 7, 0.0),
    ("k_equals_E_8", 33, 8, 8, 0, True, 1.0, 8, 0.0),
    ("softmax_no_renorm", 40, 64, 4, 0, False, 1.0, 9, 0.0),
    ("sigmoid_no_renorm", 40, 64, 4, 1, False, 1.0, 10, 0.0),
    ("max_1024x32", 64, 1024, 32, 1, True, 2.5, 11, 0.0),
]


def _logits(T, E, seed, zipf):
    if zipf:
        return synth.biased_logits(seed, synth.TID_LOGITS, T, synth.zipf_log_bias(E, zipf))
    return synth.normal_f32(seed, synth.TID_LOGITS, (T, E))


@pytest.mark.parametrize("case", ROUTE_CASES, ids=[c[0] for c in ROUTE_CASES])
def test_route_topk(case):
    name, T, E, k, score, renorm, rsf, seed, zipf = case
    logits = _logits(T, E, seed, zipf)
    ids, w = moe.moe_route_topk(dev(logits), k, score, renorm, rsf)
    torch.cuda.synchronize()
    ref_ids, ref_w = oracle.route(logits, k, score, renorm, rsf)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert rel_fro(w.cpu().numpy(), ref_w) < W_TOL


def test_route_ties_use_lower_id():
    # logits on a coarse grid: many exact ties at the top-k boundary
    T, E, k = 256, 64, 8
    logits = (np.floor(synth.normal_f32(12, 1, (T, E)) * 2.0) / 2.0).astype(np.float32)
    ids, w = moe.moe_route_topk(dev(logits), k, 1, True, 2.5)
    ref_ids, ref_w = oracle.route(logits, k, 1, True, 2.5)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert rel_fro(w.cpu().numpy(), ref_w) < W_TOL


def test_route_empty():
    ids, w = moe.moe_route_topk(torch.zeros((0, 8), dtype=torch.float32, device="cuda"), 2)
    assert ids.shape == (0, 2)


def _ids(T, E, k, seed, zipf=0.0):
    return oracle.route(_logits(T, E, seed, zipf), k, 0, True, 1.0)[0]


def _check_permute(ids, E, E_l, emap, H=0, seed=0):
    T, k = ids.shape
    R_pad = configs.permuted_rows(T, k)
    x = synth.normal_bf16(seed, 0, (T, H)) if H else None
    x_perm = None
    if H:
        x_perm = torch.full((R_pad, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    r = moe.moe_permute(dev(ids), E, E_l, None if emap is None else dev(emap),
                        None if x is None else dev_bf16(x), R_pad, x_perm=x_perm)
    torch.cuda.synchronize()
    ref_map, ref_off, _ = oracle.permute(ids, E, E_l, emap)
    assert np.array_equal(r["map"].cpu().numpy(), ref_map)
    assert np.array_equal(r["offsets"].cpu().numpy(), ref_off)
    R_l = int(ref_off[-1])
    inv = r["inv"].cpu().numpy()
    want_inv = np.full(R_pad, -1, dtype=np.int64)
    flat = ref_map.reshape(-1)
    want_inv[flat[flat >= 0]] = np.nonzero(flat >= 0)[0]
    assert np.array_equal(inv, want_inv)
    if H:
        got = host_bf16_bits(r["x_perm"])
        assert np.array_equal(got[:R_l], x[want_inv[:R_l] // k])
        # rows past the local routes are not written
        assert np.all(got[R_l:] == host_bf16_bits(torch.tensor([float("nan")],
                                                               dtype=torch.bfloat16))[0])


@pytest.mark.parametrize("T,E,k,H,zipf", [(16, 8, 2, 128, 0.0), (4096, 8, 2, 512, 1.1),
                                          (2048, 256, 8, 256, 0.0), (16384, 256, 8, 0, 0.0),
                                          (100, 1024, 16, 64, 0.0)])
def test_permute_all_local(T, E, k, H, zipf):
    _check_permute(_ids(T, E, k, 20 + T, zipf), E, E, None, H, seed=T)


@pytest.mark.parametrize("T", [1, 8, 64, 1000])
def test_permute_ep_rank_map(T):
    cfg = configs.EP_DECODE
    ids = oracle.route(synth.normal_f32(400 + T, 1, (T, cfg.E)), cfg.k, 1, True, 2.5)[0]
    _check_permute(ids, cfg.E, cfg.El, configs.expert_map(cfg), 7168, seed=T)


def test_permute_scattered_map_and_all_nonlocal():
    E, E_l = 64, 10
    rng = np.random.default_rng(5)
    emap = np.full(E, -1, dtype=np.int32)
    emap[rng.choice(E, E_l, replace=False)] = rng.permutation(E_l).astype(np.int32)
    ids = _ids(300, E, 6, 51)
    _check_permute(ids, E, E_l, emap, 128, seed=3)
    none = np.full(E, -1, dtype=np.int32)
    none[63] = 0  # one local expert that the ids below never name
    ids2 = np.array([[0, 1], [2, 3]], dtype=np.int32)
    _check_permute(ids2, E, 1, none, 64, seed=4)


@pytest.mark.parametrize("T", [50, 3000])  # one workgroup; 12 of them
def test_permute_out_of_range_ids_are_dropped(T):
    E = 16
    ids = _ids(T, E, 4, 61)
    bad = ids.copy()
    bad[3, 1] = 99
    bad[10, 0] = -5
    bad[T - 1, 3] = 1 << 30
    r = moe.moe_permute(dev(bad), E, E)
    m = r["map"].cpu().numpy()
    assert m[3, 1] == -1 and m[10, 0] == -1 and m[T - 1, 3] == -1
    # the rest equals the oracle with those routes sent to a non-local expert
    emap = np.concatenate([np.arange(E, dtype=np.int32), np.array([-1], dtype=np.int32)])
    fixed = bad.copy()
    fixed[3, 1] = E
    fixed[10, 0] = E
    fixed[T - 1, 3] = E
    ref_map, ref_off, _ = oracle.permute(fixed, E + 1, E, emap)
    assert np.array_equal(m, ref_map)
    assert np.array_equal(r["offsets"].cpu().numpy(), ref_off)


def test_permute_empty():
    r = moe.moe_permute(torch.zeros((0, 8), dtype=torch.int32, device="cuda"), 256, 256)
    assert np.all(r["offsets"].cpu().numpy() == 0)


ROUTE_PERMUTE_CASES = [
    # name, T, E, E_l (None: all local), k, score, renormalize, rsf, seed
    ("decode_1_ep_rank", 1, 256, "ep", 8, 1, True, 2.5, 500),
    ("decode_8_ep_rank", 8, 256, "ep", 8, 1, True, 2.5, 501),
    ("decode_16_ep_rank", 16, 256, "ep", 8, 1, True, 2.5, 502),
    ("ragged_13x100_top5", 13, 100, None, 5, 0, True, 1.0, 503),
    ("max_16x1024_top32", 16, 1024, None, 32, 1, True, 2.5, 504),
    ("mixtral_16x8_top2_no_renorm", 16, 8, None, 2, 0, False, 1.0, 505),
    # past one workgroup's batch: the two kernels
    ("two_kernels_17", 17, 256, "ep", 8, 1, True, 2.5, 506),
    ("two_kernels_64", 64, 256, "ep", 8, 1, True, 2.5, 508),
    ("two_kernels_2048", 2048, 256, None, 8, 1, True, 2.5, 507),
]


@pytest.mark.parametrize("case", ROUTE_PERMUTE_CASES, ids=[c[0] for c in ROUTE_PERMUTE_CASES])
def test_route_permute(case):
    """moe_route_permute equals the router and the permute of the oracle:
    ids, map, offsets and inverse map bit-exact, weights to W_TOL; the R_pad
    tail of inv is -1."""
    name, T, E, El, k, score, renorm, rsf, seed = case
    emap = None
    E_l = E
    if El == "ep":
        cfg = configs.EP_DECODE
        emap, E_l = configs.expert_map(cfg), cfg.El
    logits = synth.normal_f32(seed, synth.TID_LOGITS, (T, E))
    R_pad = configs.permuted_rows(T, k) + 37
    inv = torch.full((R_pad,), 12345, dtype=torch.int32, device="cuda")
    r = moe.moe_route_permute(dev(logits), k, score, renorm, rsf, E_l,
                              None if emap is None else dev(emap), R_pad, inv=inv)
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


def test_route_permute_matches_separate_calls_with_ties():
    # coarse logits (exact ties at the top-k boundary) on a decode batch: the
    # merged kernel gives the bits of the two separate calls
    T, E, k = 12, 64, 8
    logits = dev((np.floor(synth.normal_f32(13, 1, (T, E)) * 2.0) / 2.0).astype(np.float32))
    r = moe.moe_route_permute(logits, k, 1, True, 2.5)
    ids, w = moe.moe_route_topk(logits, k, 1, True, 2.5)
    p = moe.moe_permute(ids, E)
    torch.cuda.synchronize()
    for a, b in [(r["topk_ids"], ids), (r["topk_weights"], w), (r["map"], p["map"]),
                 (r["offsets"], p["offsets"]), (r["inv"], p["inv"])]:
        assert torch.equal(a, b)


def test_route_permute_empty():
    r = moe.moe_route_permute(torch.zeros((0, 32), dtype=torch.float32, device="cuda"), 4)
    torch.cuda.synchronize()
    assert np.all(r["offsets"].cpu().numpy() == 0)
