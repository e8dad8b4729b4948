"""The layer captured into a HIP graph and replayed.

The C ABI allocates nothing and never waits on the host, so a caller can
capture a whole layer (route, permute, GEMMs with split reductions,
finalize).  Every replay must give the eager result bit for bit, also with
eager work and synchronizations between replays and after the inputs change
in place."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_scan_amd as moe
from synth import configs

from gpu_util import dev, dev_bf16, host_bf16_bits, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("T", [1, 8, 64])
def test_decode_layer_graph_replays_match_eager(T):
    base = configs.EP_DECODE
    cfg = base.with_T(T)
    w = configs.make_weights(base)
    W1, W2 = moe.Weights(dev_bf16(w["w1"])), moe.Weights(dev_bf16(w["w2"]))
    emap = dev(configs.expert_map(cfg))
    draws = [configs.make_activations(cfg, seed=configs.EP_DECODE_DRAW_SEED0 + d) for d in range(3)]
    x = dev_bf16(draws[0][0])
    logits = dev(draws[0][1])
    R_pad = moe.moe_permuted_rows(T, cfg.k)
    nbytes = moe.moe_workspace_size(T, cfg.k, cfg.E, cfg.El, cfg.H, cfg.I)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    y = torch.empty((R_pad, cfg.H), dtype=torch.bfloat16, device="cuda")
    ew = torch.empty((T, cfg.k), dtype=torch.bfloat16, device="cuda")
    m = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    out = torch.empty((T, cfg.H), dtype=torch.bfloat16, device="cuda")

    def layer():
        moe.moe_fused_experts_unfinalized(logits, x, W1, W2, cfg.k, cfg.score, cfg.renormalize,
                                          cfg.rsf, expert_map=emap, R_pad=R_pad, workspace=ws,
                                          gemm2_permuted=y, expert_weights=ew, map=m)
        moe.moe_finalize(y, ew, m, out=out)

    def eager(d):
        x.copy_(dev_bf16(draws[d][0]))
        logits.copy_(dev(draws[d][1]))
        layer()
        torch.cuda.synchronize()
        return host_bf16_bits(out).copy(), m.cpu().numpy().copy()

    want = [eager(d) for d in range(3)]
    layer()  # warm
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()
    for rep in range(6):
        d = rep % 3
        x.copy_(dev_bf16(draws[d][0]))
        logits.copy_(dev(draws[d][1]))
        g.replay()
        torch.cuda.synchronize()
        got_out, got_m = host_bf16_bits(out), m.cpu().numpy()
        assert np.array_equal(got_m, want[d][1]), f"replay {rep}: map differs"
        assert np.array_equal(got_out, want[d][0]), f"replay {rep}: output differs"
        # eager work between replays
        scratch = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        del scratch
