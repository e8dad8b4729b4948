"""The deferred entry point that allocates nothing (its scratch is the
library's static device array) against the workspace form, through the C ABI.

Two calls in a row on one device, the second with a smaller input, at the
expert-parallel decode shape (H 7168, I 2048, 256 experts, 32 local, top-8)
and at a small shape: the permute map and the bf16 routing weights bit-exact,
every local route's gemm2_permuted row and the finalized output within the
1e-2 bar per row; a repeated call gives the same bits; a problem too large
for the static scratch is rejected on the host."""
import gc

import numpy as np
import pytest
import torch

import mixture_experts_layer_scan_amd as moe
from synth import configs

from gpu_util import dev, dev_bf16, host_bf16_bits, host_f64, need_gpu, per_row_rel

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _compare(cfg, W1, W2, emap, seed):
    x, logits = configs.make_activations(cfg, seed=seed)
    ld, xd = dev(logits), dev_bf16(x)
    args = (ld, xd, W1, W2, cfg.k, cfg.score, cfg.renormalize, cfg.rsf)
    kw = {"expert_map": emap}
    print(f"no-alloc vs workspace form: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} "
          f"E_l={cfg.El} k={cfg.k} seed={seed}", flush=True)
    y_ref, w_ref, m_ref = moe.moe_fused_experts_unfinalized(*args, **kw)
    y, w, m = moe.moe_fused_experts_unfinalized_noalloc(*args, **kw)
    y2, w2, m2 = moe.moe_fused_experts_unfinalized_noalloc(*args, **kw)
    out_ref = moe.moe_finalize(y_ref, w_ref, m_ref)
    out = moe.moe_finalize(y, w, m)
    torch.cuda.synchronize()
    mm = m.cpu().numpy()
    assert np.array_equal(mm, m_ref.cpu().numpy())
    assert np.array_equal(host_bf16_bits(w), host_bf16_bits(w_ref))
    sel = mm[mm >= 0]
    assert np.array_equal(host_bf16_bits(y2)[sel], host_bf16_bits(y)[sel]), "repeat differs"
    assert np.array_equal(m2.cpu().numpy(), mm)
    if sel.size:
        e_y = per_row_rel(host_f64(y, sel), host_f64(y_ref, sel))
        assert e_y.max() < TOL
    e_o = per_row_rel(host_f64(out), host_f64(out_ref))
    assert e_o.max() < TOL
    return int(sel.size)


def test_noalloc_ep_decode_two_calls():
    base = configs.EP_DECODE
    w = configs.make_weights(base)
    W1, W2 = moe.Weights(dev_bf16(w["w1"])), moe.Weights(dev_bf16(w["w2"]))
    emap = dev(configs.expert_map(base))
    routes = 0
    for T, seed in ((64, 500), (8, 501)):   # the second call is smaller
        routes += _compare(base.with_T(T), W1, W2, emap, seed)
    assert routes > 0


def test_noalloc_small_two_calls():
    cfg = configs.MoeConfig("noalloc_small", T=40, H=512, I=256, E=16, k=4,
                            score=configs.SIGMOID, renormalize=True, rsf=2.5, seed=31)
    w = configs.make_weights(cfg)
    W1, W2 = moe.Weights(dev_bf16(w["w1"])), moe.Weights(dev_bf16(w["w2"]))
    _compare(cfg, W1, W2, None, 600)
    _compare(cfg.with_T(5), W1, W2, None, 601)


def test_noalloc_rejects_oversized_problem():
    """A problem whose scratch (without the GEMM partials) exceeds the static
    array fails before anything is enqueued."""
    T, H, I, E, k = 8192, 7168, 2048, 8, 8
    lg = torch.zeros((T, E), dtype=torch.float32, device="cuda")
    x = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    W1 = moe.Weights(torch.zeros((E, 2 * I, H), dtype=torch.bfloat16, device="cuda"))
    W2 = moe.Weights(torch.zeros((E, H, I), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(RuntimeError, match="static scratch"):
        moe.moe_fused_experts_unfinalized_noalloc(lg, x, W1, W2, k)
