#!/usr/bin/env python3
"""Benchmark of the fused MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]

One step is the whole hot path on one batch of synthetic input already
resident in HBM: route -> permute (map, offsets, row gather) -> grouped GEMM1
with SiLU(gate)*up -> grouped GEMM2 -> finalize.  The default workload is the
Mixtral-8x7B-shaped prefill layer (4096 tokens, hidden 4096, intermediate
14336, 8 experts, top-2, Zipf(1.1)-biased routing), random bf16 weights.

Prints one JSON line: tokens/s (value), algorithmic TFLOP/s, the roofline of
the dominant kernel (grouped GEMM1) from HIP events recorded around each of its
launches on the launching stream, and the CPU oracle timed on a bounded sample
of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused-MoE layer tokens/s and TFLOP/s (% MFMA or HBM peak), 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_DIR = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="mixtral8x7b_prefill_4096tok")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="before the warm-up, run one device-to-device copy of this many MiB "
                        "(a plain copy kernel of known size, to scale HBM byte counters)")
    return p.parse_args()


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "mixture_experts_layer_scan_amd", "csrc", "gemm.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per GEMM1 launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy kernel), or None when it is
    missing or was taken on a different gemm.hip."""
    path = os.path.join(TRAFFIC_DIR, f"gemm_hbm_traffic_{workload}.txt")
    try:
        with open(path) as f:
            kv = dict(l.strip().split("=", 1) for l in f
                      if "=" in l and not l.lstrip().startswith("#"))
    except OSError:
        return None
    if kv.get("gemm_source_sha256_16") != gemm_source_hash() or kv.get("workload") != workload:
        return None
    return float(kv["gemm1_hbm_bytes_per_launch"])


def cpu_baseline(cfg, x, logits, w, target_s: float):
    import oracle
    W1, W2 = oracle.Weights(w["w1"]), oracle.Weights(w["w2"])
    kw = dict(expert_map=None, shared_I=cfg.shared_I, ws1=w.get("ws1"), ws2=w.get("ws2"))
    # warm-up touch of the weight pages with one token
    oracle.moe_tokens(x, logits, W1, W2, cfg.I, cfg.k, cfg.score, cfg.renormalize, cfg.rsf,
                      tokens=[0], **kw)
    n = max(oracle.num_threads(), 1)
    t0 = time.perf_counter()
    oracle.moe_tokens(x, logits, W1, W2, cfg.I, cfg.k, cfg.score, cfg.renormalize, cfg.rsf,
                      tokens=list(range(n)), **kw)
    dt = time.perf_counter() - t0
    total_tok, total_s = n, dt
    if dt < target_s:
        m = int(min(cfg.T - n, max(n, (target_s - dt) / dt * n)))
        m = max(n, m // n * n)
        t0 = time.perf_counter()
        oracle.moe_tokens(x, logits, W1, W2, cfg.I, cfg.k, cfg.score, cfg.renormalize, cfg.rsf,
                          tokens=list(range(n, n + m)), **kw)
        total_s += time.perf_counter() - t0
        total_tok += m
    return {"value": total_tok / total_s, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"first {total_tok} of {cfg.T} tokens of the same workload, float64 "
                      f"per-token per-expert MLP, {total_s:.1f} s wall"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the layer's "
              f"multi-GPU sharding is a design note, not a measured path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixture_experts_layer_scan_amd as moe
    from synth import configs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    cfg = configs.ALL[args.workload]
    if cfg.deferred or cfg.mxfp4:
        print(f"workload {cfg.name} is a parity-test configuration; bench covers the "
              f"finalized bf16 layers", file=sys.stderr)
        sys.exit(2)

    x, logits = configs.make_activations(cfg)
    w = configs.make_weights(cfg)

    def to_bf16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

    xd, ld = to_bf16(x), torch.from_numpy(logits).cuda()
    W1, W2 = moe.Weights(to_bf16(w["w1"])), moe.Weights(to_bf16(w["w2"]))
    emap = configs.expert_map(cfg)
    emap_d = None if emap is None else torch.from_numpy(emap).cuda()
    T, H, I, k, E, El = cfg.T, cfg.H, cfg.I, cfg.k, cfg.E, cfg.El
    R_pad = moe.moe_permuted_rows(T, k)
    dev = "cuda"
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    pmap = torch.empty((T, k), dtype=torch.int32, device=dev)
    offsets = torch.empty((El + 1,), dtype=torch.int32, device=dev)
    x_perm = torch.empty((R_pad, H), dtype=torch.bfloat16, device=dev)
    h = torch.empty((R_pad, I), dtype=torch.bfloat16, device=dev)
    y = torch.empty((R_pad, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    shared = None
    if cfg.shared_I:
        WS1 = moe.Weights(to_bf16(w["ws1"])[None])
        WS2 = moe.Weights(to_bf16(w["ws2"])[None])
        off_s = torch.tensor([0, T], dtype=torch.int32, device=dev)
        hs = torch.empty((T, cfg.shared_I), dtype=torch.bfloat16, device=dev)
        shared = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    stages = ["route", "permute", "gemm1", "gemm2", "shared", "finalize"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        moe.moe_route_topk(ld, k, cfg.score, cfg.renormalize, cfg.rsf, ids, wts, stream)
        mark(1)
        moe.moe_permute(ids, E, El, emap_d, xd, R_pad, pmap, offsets, None, x_perm,
                        want_inv=False, stream=stream)
        mark(2)
        moe.moe_grouped_gemm1_act(x_perm, offsets, W1, I, h, stream=stream)
        mark(3)
        moe.moe_grouped_gemm2(h, offsets, W2, H, y, stream=stream)
        mark(4)
        if cfg.shared_I:
            moe.moe_grouped_gemm1_act(xd, off_s, WS1, cfg.shared_I, hs, stream=stream)
            moe.moe_grouped_gemm2(hs, off_s, WS2, H, shared, stream=stream)
        mark(5)
        moe.moe_finalize(y, wts, pmap, 1.0, shared, out, stream=stream)
        mark(6)

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    stage_ms = {s: float(np.mean([events[i][j].elapsed_time(events[i][j + 1])
                                  for i in range(args.steps)]))
                for j, s in enumerate(stages)}
    if not cfg.shared_I:
        del stage_ms["shared"]
    counts = np.diff(offsets.cpu().numpy())
    R_l = int(counts.sum())
    flops_gemm1 = 2.0 * R_l * H * (2 * I)
    flops_gemm2 = 2.0 * R_l * I * H
    flops_shared = 6.0 * T * H * cfg.shared_I
    flops_step = flops_gemm1 + flops_gemm2 + flops_shared
    ms_per_step = elapsed / args.steps * 1e3
    gemm1_s = stage_ms["gemm1"] * 1e-3
    achieved = flops_gemm1 / gemm1_s / 1e12
    traffic = measured_traffic(cfg.name)

    result = {
        "metric": METRIC,
        "value": T * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/sqrt(fan_in)) random weights)",
        "config": {"workload": cfg.name, "tokens": T, "hidden": H, "intermediate": I,
                   "experts": E, "local_experts": El, "top_k": k,
                   "shared_intermediate": cfg.shared_I,
                   "routing": ("softmax" if cfg.score == 0 else "sigmoid") +
                              (f" top-{k} renormalized") + (f", rsf {cfg.rsf}" if cfg.rsf != 1 else "") +
                              (f", Zipf({cfg.zipf_s}) logit bias" if cfg.zipf_s else "")},
        "tflops": flops_step / (ms_per_step * 1e-3) / 1e12,
        "mfma_frac_layer": flops_step / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "stages_ms": stage_ms,
        "expert_rows": counts.tolist() if len(counts) <= 16 else
                       {"min": int(counts.min()), "max": int(counts.max()), "mean": float(counts.mean())},
        "roofline": {"kernel": "grouped_gemm1_act", "bound": "mfma", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic,
                     "algorithmic_flop_per_launch": flops_gemm1},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        del xd, ld, W1, W2, x_perm, h, y, out
        result["cpu_baseline"] = cpu_baseline(cfg, x, logits, w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
