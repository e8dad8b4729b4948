"""GPU parity of the fused tail (finalize + shared add + residual add + RMSNorm)
against the oracle: the new residual and the normalized output within 1e-2
relative Frobenius error; tokens with no local route; determinism."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_scan_amd as moe
import oracle
import synth
from synth import configs

from gpu_util import dev, dev_bf16, host_bf16_bits, host_f64, need_gpu, rel_fro

pytestmark = pytest.mark.gpu

TOL = 1e-2

CASES = [
    # name, T, E, E_l (None: all local), k, H, weights dtype, shared, rsf_fin
    ("ep_decode_bf16", 64, 256, 32, 8, 7168, torch.bfloat16, False, 1.0),
    ("ep_single_token", 1, 256, 32, 8, 7168, torch.bfloat16, False, 1.0),
    ("deepseek_shared_f32", 96, 256, None, 8, 7168, torch.float32, True, 1.0),
    ("mixtral_rsf", 300, 8, None, 2, 4096, torch.float32, False, 0.5),
    ("small_h", 17, 8, None, 2, 136, torch.float32, True, 1.0),
]


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_finalize_add_rmsnorm(case):
    name, T, E, E_l, k, H, wdt, with_shared, rsf_fin = case
    seed = T + H + k
    logits = synth.normal_f32(seed, 1, (T, E))
    ids, w = oracle.route(logits, k, 1, True, 2.5)
    emap = configs.expert_map(configs.EP_DECODE) if E_l is not None else None
    m, off, _ = oracle.permute(ids, E, E_l or E, emap)
    R_pad = configs.permuted_rows(T, k)
    y = synth.normal_bf16(seed, 2, (R_pad, H))
    y[int(off[-1]):] = 0x7FC0  # never read
    shared = synth.normal_bf16(seed, 5, (T, H)) if with_shared else None
    res = synth.normal_bf16(seed, 6, (T, H), std=4.0)
    gamma = synth.normal_bf16(seed, 7, (H,), mean=1.0, std=0.2)
    w_dev = dev(w.astype(np.float32))
    if wdt == torch.bfloat16:
        w_dev = w_dev.to(torch.bfloat16)
    w_used = host_f64(w_dev)
    res_dev = dev_bf16(res)
    out, res_new = moe.moe_finalize_add_rmsnorm(dev_bf16(y), w_dev, dev(m), res_dev, dev_bf16(gamma),
                                                1e-6, rsf_fin,
                                                None if shared is None else dev_bf16(shared))
    torch.cuda.synchronize()
    ref_res, ref_out = oracle.finalize_add_rmsnorm(y, w_used, m, res, gamma, 1e-6, rsf_fin, shared)
    assert res_new.data_ptr() == res_dev.data_ptr()
    assert rel_fro(host_f64(res_new), ref_res) < TOL
    got = host_f64(out)
    assert np.all(np.isfinite(got))
    assert rel_fro(got, ref_out) < TOL
    # the same bits again from the same inputs
    res2 = dev_bf16(res)
    out2, _ = moe.moe_finalize_add_rmsnorm(dev_bf16(y), w_dev, dev(m), res2, dev_bf16(gamma), 1e-6,
                                           rsf_fin, None if shared is None else dev_bf16(shared))
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(out2), host_bf16_bits(out))
