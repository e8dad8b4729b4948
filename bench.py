#!/usr/bin/env python3
"""Benchmark of the fused MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME] [--tokens T]
                    [--activation silu|gelu] [--activation-clamp C] [--top-k K]
                    [--router-weight-on-input] [--chunk-tokens N] [--batched-max-tokens M]
                    [--fused-tail] [--graph]

One step is the whole hot path on one batch of synthetic input already
resident in HBM: route -> permute (map, offsets, row gather) -> grouped GEMM1
with SiLU(gate)*up -> grouped GEMM2 (-> shared expert) -> finalize.  The
default workload is the Mixtral-8x7B-shaped prefill layer (4096 tokens, hidden
4096, intermediate 14336, 8 experts, top-2, Zipf(1.1)-biased routing), random
bf16 weights.  The other workloads:
  deepseekv3_routed_shared_2048tok   256 experts, top-8 sigmoid, shared expert
  deepseekv3_mxfp4_2048tok           the same shape with MXFP4 expert weights
  deepseekv3_fp8_2048tok             the same shape (routed experts only) in FP8 E4M3:
                                     per-channel weight scales, per-token activation
                                     scales (quantize -> dispatch -> FP8 GEMMs)
  mixtral8x7b_fp8_prefill_4096tok    the Mixtral shape in FP8 E4M3
  deepseekv3_mxfp4_x2act_2048tok     MXFP4 weights with the bf16 activations carried as two FP8
                                     terms, scale * (q1 + q2 / 16), through the FP8 x e2m1
                                     matrix cores (near-bf16 activation precision)
  deepseekv3_mxfp4_fp8act_2048tok    MXFP4 weights with FP8 activations per token (FP8 x e2m1
                                     on the matrix cores, E8M0 block scales applied by them)
  deepseekv3_fp8block_2048tok        the DeepSeek-V3 routed shape in blockwise FP8: one weight
                                     scale per 128 x 128 block, one activation scale per token
                                     and 128-element group
  ep_rank3of8_decode                 one expert-parallel rank's 32 experts at a
                                     decode batch (--tokens 1, 8 or 64), deferred
                                     form followed by the separate finalize; the
                                     steps cycle through 16 routing draws and a
                                     512 MiB read evicts L2 and the MALL before
                                     each step (outside the timed events)

Variants of a workload (each named in config.workload): GELU instead of SiLU,
an activation clamp, another top_k, the routing weight applied to the input
rows (top_k 1), activation chunking (the layer over consecutive chunks of N
tokens with buffers sized for one chunk; every chunk re-streams the weights of
its experts), and the batched experts format (rows laid out per local expert
with a capacity of M tokens each).

Prints one JSON line: tokens/s (value), algorithmic TFLOP/s, the roofline of
the dominant kernel (grouped GEMM1) from HIP events recorded around each of its
launches on the launching stream -- against the bf16 MFMA peak when its
algorithmic flops take longer there than its algorithmic bytes take at the HBM
peak, else against the HBM peak -- and the CPU oracle timed on a bounded
sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import ctypes
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
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_DIR = os.path.join(ROOT, "profiles")
FLUSH_BYTES = 512 << 20     # > L2 (8 x 4 MiB) + MALL (256 MiB)
HOST_AHEAD_CYCLES = 2_000_000  # GPU spin before each decode step (outside the events)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3000,
                   help="timed steps of the throughput pass (the default keeps the GPU busy for "
                        "several seconds); the per-stage pass runs the first min(steps, 100)")
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="mixtral8x7b_prefill_4096tok")
    p.add_argument("--tokens", type=int, default=64,
                   help="decode batch of the expert-parallel decode workload (1, 8 or 64)")
    p.add_argument("--graph", action="store_true",
                   help="replay the layer as a captured HIP graph (one per input batch); "
                        "the stage breakdown is then not available")
    p.add_argument("--fused-tail", action="store_true",
                   help="end the step with the fused tail (finalize + shared add + residual add "
                        "+ the next layer's RMSNorm) instead of the plain finalize")
    p.add_argument("--activation", choices=["silu", "gelu"], default="silu")
    p.add_argument("--activation-clamp", type=float, default=0.0,
                   help="> 0: clamp the gate from above and the up value on both sides first")
    p.add_argument("--top-k", type=int, default=0, help="override the workload's top_k")
    p.add_argument("--router-weight-on-input", action="store_true",
                   help="apply the routing weights to the input rows (top_k 1 only)")
    p.add_argument("--chunk-tokens", type=int, default=0,
                   help="run the layer over chunks of this many tokens")
    p.add_argument("--batched-max-tokens", type=int, default=0,
                   help="use the batched experts format with this capacity per local expert")
    p.add_argument("--gather-kernel", action="store_true",
                   help="gather the permuted rows with the permute's own kernel wherever GEMM1 "
                        "would read them through the inverse map")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="before the warm-up, run one device-to-device copy of this many MiB "
                        "(a plain copy kernel of known size, to scale HBM byte counters)")
    return p.parse_args()


def gemm_source_hash() -> str:
    """Hash of the GEMM kernels' sources (the tiled kernels and the decode kernel)."""
    h = hashlib.sha256()
    for name in ("gemm.hip", "decode_gemm.hip"):
        with open(os.path.join(ROOT, "mixture_experts_layer_scan_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per GEMM1 launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy kernel), or None when it is
    missing or was taken on different GEMM sources."""
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


def gemm_work(cfg, counts, gemm: int):
    """Algorithmic flops and HBM bytes of one grouped-GEMM launch: the weights
    of the experts that received rows (E8M0 scales included), the input rows
    read once, the output rows written once."""
    counts = np.asarray(counts, dtype=np.int64)
    R_l, touched = int(counts.sum()), int((counts > 0).sum())
    if gemm == 1:
        N, K, out_cols = 2 * cfg.I, cfg.H, cfg.I
    else:
        N, K, out_cols = cfg.H, cfg.I, cfg.H
    if cfg.mxfp4:
        w_bytes_per_expert = N * (K // 2 + K // 32)
    elif cfg.fp8_block:
        w_bytes_per_expert = N * K + (N // 128) * (K // 128) * 4   # codes + one scale per block
    elif cfg.fp8:
        w_bytes_per_expert = N * (K + 4)     # codes + one fp32 scale per channel
    else:
        w_bytes_per_expert = N * K * 2
    # fp8 rows carry a scale; two-term rows hold 2K codes
    in_bytes = (R_l * (K + 4 * (K // 128)) if cfg.fp8_block else R_l * (K + 4) if cfg.fp8
                else R_l * (2 * K + 4) if cfg.fp8x2 else R_l * K * 2)
    flops = 2.0 * R_l * N * K
    nbytes = float(touched * w_bytes_per_expert + in_bytes + R_l * out_cols * 2)
    return flops, nbytes


def cpu_baseline(cfg, draws, w, target_s: float, variant=None):
    """The oracle as it stands, on all host cores, on a bounded sample of the
    workload's tokens (draw after draw, chunk after chunk) until about
    target_s seconds of CPU work."""
    import oracle
    if cfg.mxfp4:
        W1, W2 = oracle.Weights(w["w1_q"], w["w1_s"]), oracle.Weights(w["w2_q"], w["w2_s"])
    elif cfg.fp8_block:
        W1 = oracle.Weights(w["w1_q"], w["w1_s"], block=True)
        W2 = oracle.Weights(w["w2_q"], w["w2_s"], block=True)
    elif cfg.fp8:
        W1 = oracle.Weights(w["w1_q"], w["w1_s"].reshape(-1))
        W2 = oracle.Weights(w["w2_q"], w["w2_s"].reshape(-1))
    else:
        W1, W2 = oracle.Weights(w["w1"]), oracle.Weights(w["w2"])
    from synth import configs
    kw = dict(expert_map=configs.expert_map(cfg), shared_I=cfg.shared_I, ws1=w.get("ws1"),
              ws2=w.get("ws2"),
              fp8="x2" if cfg.fp8x2 else "block" if cfg.fp8_block else cfg.fp8,
              **(variant or {}))

    def run(x, logits, toks):
        oracle.moe_tokens(x, logits, W1, W2, cfg.I, cfg.k, cfg.score, cfg.renormalize, cfg.rsf,
                          tokens=toks, **kw)

    run(draws[0][0], draws[0][1], [0])  # page-touch warm-up
    n = max(oracle.num_threads(), 1)
    chunk, total_tok, total_s, n_draws = n, 0, 0.0, 0
    while total_s < target_s:
        x, logits = draws[n_draws % len(draws)]
        T = x.shape[0]
        n_draws += 1
        for start in range(0, T, chunk):
            toks = list(range(start, min(T, start + chunk)))
            t0 = time.perf_counter()
            run(x, logits, toks)
            dt = time.perf_counter() - t0
            total_tok += len(toks)
            total_s += dt
            if total_s >= target_s:
                break
            if dt < target_s / 8:
                chunk *= 2
        if n_draws > 200000:  # (a bound on the loop; the time target ends it first)
            break
    if len(draws) > 1:
        where = f"{total_tok} tokens from {n_draws} routing draws of {cfg.T} tokens"
    elif n_draws > 1:
        where = f"{total_tok} tokens ({n_draws} passes over the {cfg.T} tokens)"
    else:
        where = f"first {total_tok} of {cfg.T} tokens"
    return {"value": total_tok / total_s, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{where} of the same workload, float64 per-token per-expert MLP, "
                      f"{total_s:.1f} s wall"}


class TimingEvent:
    """A HIP event used only to time GPU work: created with
    hipEventDisableSystemFence, so recording it skips the system-scope fence
    (a cache write-back and invalidation) that the default event performs,
    which idles the GPU before the next kernel and leaves it cold caches.  The
    interface is torch.cuda.Event's record / elapsed_time; the host
    synchronizes with torch.cuda.synchronize() before reading it."""

    _hip = None
    _FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        if TimingEvent._hip is None:
            TimingEvent._hip = ctypes.CDLL("libamdhip64.so")
        self._e = ctypes.c_void_p()
        self._call("hipEventCreateWithFlags", ctypes.byref(self._e), ctypes.c_uint(self._FLAGS))

    def _call(self, fn, *a):
        rc = getattr(TimingEvent._hip, fn)(*a)
        if rc != 0:
            raise RuntimeError(f"{fn} failed ({rc})")

    def record(self, stream=None):
        import torch
        s = (stream if stream is not None else torch.cuda.current_stream()).cuda_stream
        self._call("hipEventRecord", self._e, ctypes.c_void_p(s))

    def elapsed_time(self, end) -> float:
        ms = ctypes.c_float()
        self._call("hipEventElapsedTime", ctypes.byref(ms), self._e, end._e)
        return ms.value

    def __del__(self):
        if self._e:
            TimingEvent._hip.hipEventDestroy(self._e)


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
    if args.workload not in configs.ALL:
        print(f"unknown workload {args.workload}; one of {sorted(configs.ALL)}", file=sys.stderr)
        sys.exit(2)
    cfg = configs.ALL[args.workload]
    if args.top_k:
        import dataclasses
        cfg = dataclasses.replace(cfg, k=args.top_k)
    if args.router_weight_on_input and cfg.k != 1:
        print("--router-weight-on-input needs top_k 1 (--top-k 1)", file=sys.stderr)
        sys.exit(2)
    decode = cfg.deferred
    if decode:
        if args.tokens not in configs.EP_DECODE_BATCHES:
            print(f"--tokens must be one of {configs.EP_DECODE_BATCHES}", file=sys.stderr)
            sys.exit(2)
        cfg = cfg.with_T(args.tokens)
        draws = [configs.make_activations(cfg, seed=configs.EP_DECODE_DRAW_SEED0 + d)
                 for d in range(configs.EP_DECODE_DRAWS)]
        label = f"{cfg.name}_T{cfg.T}"
    else:
        draws = [configs.make_activations(cfg)]
        label = cfg.name
    if args.top_k:
        label += f"_top{cfg.k}"
    if args.activation != "silu":
        label += f"_{args.activation}"
    if args.activation_clamp:
        label += f"_clamp{args.activation_clamp:g}"
    if args.router_weight_on_input:
        label += "_weight_on_input"
    if args.chunk_tokens and args.chunk_tokens < cfg.T:
        label += f"_chunk{args.chunk_tokens}"
    if args.batched_max_tokens:
        label += f"_batched{args.batched_max_tokens}"
    variant = {"activation": args.activation, "clamp": args.activation_clamp,
               "weight_on_input": args.router_weight_on_input}
    w = configs.make_weights(cfg)

    def to_bf16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

    dev_draws = [(to_bf16(x), torch.from_numpy(lg).cuda()) for x, lg in draws]
    if cfg.mxfp4 or cfg.fp8 or cfg.fp8_block:
        W1 = moe.Weights(torch.from_numpy(w["w1_q"]).cuda(), torch.from_numpy(w["w1_s"]).cuda())
        W2 = moe.Weights(torch.from_numpy(w["w2_q"]).cuda(), torch.from_numpy(w["w2_s"]).cuda())
    else:
        W1, W2 = moe.Weights(to_bf16(w["w1"])), moe.Weights(to_bf16(w["w2"]))
    emap = configs.expert_map(cfg)
    emap_d = None if emap is None else torch.from_numpy(emap).cuda()
    T, H, I, k, E, El = cfg.T, cfg.H, cfg.I, cfg.k, cfg.E, cfg.El
    P = min(T, args.chunk_tokens) if args.chunk_tokens > 0 else T  # tokens per pass
    chunks = [(t0, min(P, T - t0)) for t0 in range(0, T, P)]
    Mb = args.batched_max_tokens
    R_pad = El * Mb if Mb else moe.moe_permuted_rows(P, k)
    dev = "cuda"
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    pmap = torch.empty((T, k), dtype=torch.int32, device=dev)
    offsets = torch.empty((El + 1,), dtype=torch.int32, device=dev)
    x_perm = torch.empty((R_pad, H), dtype=torch.bfloat16, device=dev)
    h = torch.empty((R_pad, I), dtype=torch.bfloat16, device=dev)
    y = torch.empty((R_pad, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    quant = cfg.fp8 or cfg.fp8x2 or cfg.fp8_block   # activations quantized inside the layer
    terms = 2 if cfg.fp8x2 else 1
    if quant:
        if Mb:
            print("FP8 workloads take the standard layout", file=sys.stderr)
            sys.exit(2)
        xq = torch.empty((T, H * terms), dtype=torch.uint8, device=dev)
        xq_perm = torch.empty((R_pad, H * terms), dtype=torch.uint8, device=dev)
        hq = torch.empty((R_pad, I * terms), dtype=torch.uint8, device=dev)
        if cfg.fp8_block:   # group-major scales, one per row and 128 elements
            xs = torch.empty((H // 128, T), dtype=torch.float32, device=dev)
            ps = torch.empty((H // 128, R_pad), dtype=torch.float32, device=dev)
            hs = torch.empty((I // 128, R_pad), dtype=torch.float32, device=dev)
        else:
            xs = torch.empty((T,), dtype=torch.float32, device=dev)
            ps = torch.empty((R_pad,), dtype=torch.float32, device=dev)
            hs = torch.empty((R_pad,), dtype=torch.float32, device=dev)
    if args.fused_tail:
        residual = to_bf16(draws[0][0])  # a residual stream of the x distribution
        gamma = torch.ones(H, dtype=torch.bfloat16, device=dev)
    shared = None
    if cfg.shared_I:
        WS1 = moe.Weights(to_bf16(w["ws1"])[None])
        WS2 = moe.Weights(to_bf16(w["ws2"])[None])
        off_s = {n: torch.tensor([0, n], dtype=torch.int32, device=dev) for _, n in chunks}
        hs = torch.empty((P, cfg.shared_I), dtype=torch.bfloat16, device=dev)
        shared = torch.empty((P, H), dtype=torch.bfloat16, device=dev)
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev) if decode else None
    flush_sum = torch.zeros((), dtype=torch.float32, device=dev)

    def evict_caches():
        # read (not write) 512 MiB: evicts L2 and the MALL without leaving
        # dirty lines whose write-back would compete with the next step
        torch.sum(flush, dim=0, out=flush_sum)
    # split-reduction scratch of the two GEMMs (used one after the other)
    ws_bytes = max(moe.moe_grouped_gemm_workspace_size(R_pad, I, True),
                   moe.moe_grouped_gemm_workspace_size(R_pad, H, False))
    split_ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    stream = torch.cuda.current_stream()

    fin_stage = "finalize_add_rmsnorm" if args.fused_tail else "finalize"
    stages = None  # set below, once the dispatch form is known
    act_kw = dict(activation=args.activation, activation_clamp=args.activation_clamp)
    w_in = args.router_weight_on_input

    counts_b = torch.empty((El,), dtype=torch.int32, device=dev)
    # bf16 passes in the standard layout: GEMM1 reads its rows from x through
    # the permute's inverse map, as the library's fused calls do (no gather kernel)
    gathered = (not quant and not Mb and not w_in and P * H * 2 <= 0xFFFFFFFF
                and not args.gather_kernel)
    # two-term rows, and one-term FP8 rows of batches up to 64 tokens: GEMM1
    # reads the quantized token rows through the inverse map too (as the
    # library's fused calls do)
    gathered_q = (quant and not cfg.fp8_block and (cfg.fp8x2 or P <= 64)
                  and P * H * terms <= 0xFFFFFFFF and not args.gather_kernel)
    inv_buf = (torch.empty((R_pad,), dtype=torch.int32, device=dev)
               if gathered or gathered_q else None)
    # a batch of at most 16 tokens routes and permutes in one launch; a bf16
    # one of at most 8 tokens and 64 routes also runs GEMM1 in that launch
    # (the library chooses: one kernel when the decode GEMM applies)
    merged = (gathered or gathered_q) and P <= 16
    fused_g1 = merged and not quant and not cfg.shared_I and P <= 8 and P * k <= 64
    first = ["route_permute"] if merged else ["route"]
    if fused_g1:
        stages = ["route_permute_gemm1", "gemm2"]
    elif quant:
        stages = (first + ["quantize"] + ([] if merged else ["permute"])
                  + ["gemm1", "quantize_h", "gemm2"])
    else:
        stages = first + ([] if merged else ["permute"]) + ["gemm1", "gemm2"]
    stages += (["shared"] if cfg.shared_I else []) + [fin_stage]

    def route_and_map(ld, sl, st):
        """Router and permute map of a small batch in one call (gathered GEMM1)."""
        moe.moe_route_permute(ld[sl], k, cfg.score, cfg.renormalize, cfg.rsf, El, emap_d, R_pad,
                              ids[sl], wts[sl], pmap[sl], offsets, inv_buf, stream=st)

    def quantize_tokens(sl, st):
        if cfg.fp8x2:
            moe.moe_quantize_fp8x2(xd_cur[0][sl], wts[sl] if w_in else None, xq[sl], xs[sl],
                                   stream=st)
        else:
            moe.moe_quantize_fp8(xd_cur[0][sl], None, wts[sl] if w_in else None, xq[sl], xs[sl],
                                 stream=st)

    def permute(sl, st):
        if cfg.fp8_block:
            moe.moe_quantize_fp8_blockwise(xd_cur[0][sl], None, xq[sl], xs[:, sl], stream=st)
            mark_cur[0]("permute")
            moe.moe_permute_fp8_blockwise(ids[sl], E, xq[sl], xs[:, sl], El, emap_d, R_pad,
                                          pmap[sl], offsets, None, xq_perm, ps, want_inv=False,
                                          stream=st)
            return
        if quant:
            quantize_tokens(sl, st)
            mark_cur[0]("permute")
            if gathered_q:
                moe.moe_permute(ids[sl], E, El, emap_d, None, R_pad, pmap[sl], offsets, inv_buf,
                                stream=st)
            else:
                moe.moe_permute_fp8(ids[sl], E, xq[sl], xs[sl], El, emap_d, R_pad, pmap[sl],
                                    offsets, None, xq_perm, ps, want_inv=False, stream=st)
            return
        if Mb:
            moe.moe_permute_batched(ids[sl], E, Mb, El, emap_d, xd_cur[0][sl], pmap[sl], counts_b,
                                    x_perm.view(El, Mb, H), wts[sl] if w_in else None, stream=st)
        elif gathered:
            moe.moe_permute(ids[sl], E, El, emap_d, None, R_pad, pmap[sl], offsets, inv_buf,
                            stream=st)
        else:
            moe.moe_permute(ids[sl], E, El, emap_d, xd_cur[0][sl], R_pad, pmap[sl], offsets, None,
                            x_perm, want_inv=False, x_weights=wts[sl] if w_in else None,
                            stream=st)

    def gemms(n, st):
        if cfg.fp8_block:
            moe.moe_grouped_gemm1_act_fp8_blockwise(xq_perm, ps, offsets, W1, I, h, stream=st,
                                                    split=False, workspace=split_ws, **act_kw)
            mark_cur[0]("quantize_h")
            moe.moe_quantize_fp8_blockwise(h, offsets[El:], hq, hs, stream=st)
            mark_cur[0]("gemm2")
            moe.moe_grouped_gemm2_fp8_blockwise(hq, hs, offsets, W2, H, y, stream=st, split=False,
                                                workspace=split_ws)
            return
        if quant and gathered_q:
            moe.moe_grouped_gemm1_act_fp8_gathered(xq[gsl[0]], xs[gsl[0]], inv_buf, k, offsets,
                                                   W1, I, terms=terms, h=h, stream=st,
                                                   split=False, workspace=split_ws, **act_kw)
        elif cfg.fp8x2:
            moe.moe_grouped_gemm1_act_fp8x2(xq_perm, ps, offsets, W1, I, h, stream=st,
                                            split=False, workspace=split_ws, **act_kw)
        if cfg.fp8x2:
            mark_cur[0]("quantize_h")
            moe.moe_quantize_fp8x2(h, None, hq, hs, row_count=offsets[El:], stream=st)
            mark_cur[0]("gemm2")
            moe.moe_grouped_gemm2_fp8x2(hq, hs, offsets, W2, H, y, stream=st, split=False,
                                        workspace=split_ws)
            return
        if cfg.fp8:
            if not gathered_q:
                moe.moe_grouped_gemm1_act_fp8(xq_perm, ps, offsets, W1, I, h, stream=st,
                                              split=False, workspace=split_ws, **act_kw)
            mark_cur[0]("quantize_h")
            moe.moe_quantize_fp8(h, None, None, hq, hs, row_count=offsets[El:], stream=st)
            mark_cur[0]("gemm2")
            moe.moe_grouped_gemm2_fp8(hq, hs, offsets, W2, H, y, stream=st, split=False,
                                      workspace=split_ws)
            return
        if Mb:
            moe.moe_grouped_gemm1_act_batched(x_perm.view(El, Mb, H), counts_b, W1, I,
                                              h.view(El, Mb, I), max_rows=n * k, stream=st,
                                              split=False, workspace=split_ws, **act_kw)
            mark_cur[0]("gemm2")
            moe.moe_grouped_gemm2_batched(h.view(El, Mb, I), counts_b, W2, H, y.view(El, Mb, H),
                                          max_rows=n * k, stream=st, split=False,
                                          workspace=split_ws)
        else:
            if gathered:
                moe.moe_grouped_gemm1_act_gathered(xd_cur[0][gsl[0]], inv_buf, k, offsets, W1, I,
                                                   h, stream=st, split=False, workspace=split_ws,
                                                   **act_kw)
            else:
                moe.moe_grouped_gemm1_act(x_perm, offsets, W1, I, h, stream=st, split=False,
                                          workspace=split_ws, **act_kw)
            mark_cur[0]("gemm2")
            moe.moe_grouped_gemm2(h, offsets, W2, H, y, stream=st, split=False,
                                  workspace=split_ws)

    xd_cur, mark_cur, gsl = [None], [None], [None]

    def route_permute(d, t0, n):
        xd, ld = dev_draws[d]
        xd_cur[0], mark_cur[0] = xd, (lambda name: None)
        sl = slice(t0, t0 + n)
        if merged:  # (the counts come from the same permute either way)
            route_and_map(ld, sl, stream)
            return
        moe.moe_route_topk(ld[sl], k, cfg.score, cfg.renormalize, cfg.rsf, ids[sl], wts[sl],
                           stream)
        permute(sl, stream)

    def chunk_counts():
        return counts_b.cpu().numpy().clip(0, Mb) if Mb else np.diff(offsets.cpu().numpy())

    def layer(d, st, mark=lambda name: None):
        """The layer on input batch d, enqueued on stream st, one pass per
        chunk; mark(name) records the start of stage `name` (None: the end)."""
        xd, ld = dev_draws[d]
        xd_cur[0], mark_cur[0] = xd, mark
        for t0, n in chunks:
            sl = slice(t0, t0 + n)
            gsl[0] = sl
            if fused_g1:
                mark("route_permute_gemm1")
                moe.moe_route_permute_gemm1_act(
                    ld[sl], xd[sl], k, W1, I, cfg.score, cfg.renormalize, cfg.rsf, emap_d, R_pad,
                    ids[sl], wts[sl], pmap[sl], offsets, inv_buf, h, stream=st, split=False,
                    workspace=split_ws, **act_kw)
                mark("gemm2")
                moe.moe_grouped_gemm2(h, offsets, W2, H, y, stream=st, split=False,
                                      workspace=split_ws)
                mark(fin_stage)
                wf = None if w_in else wts[sl]
                if args.fused_tail:
                    moe.moe_finalize_add_rmsnorm(y, wf, pmap[sl], residual[sl], gamma, 1e-6, 1.0,
                                                 None, out[sl], stream=st)
                else:
                    moe.moe_finalize(y, wf, pmap[sl], 1.0, None, out[sl], stream=st)
                continue
            if merged:
                mark("route_permute")
                route_and_map(ld, sl, st)
                if quant:
                    mark("quantize")
                    quantize_tokens(sl, st)
            else:
                mark("route")
                moe.moe_route_topk(ld[sl], k, cfg.score, cfg.renormalize, cfg.rsf, ids[sl],
                                   wts[sl], st)
                mark("quantize" if quant else "permute")
                permute(sl, st)
            mark("gemm1")
            gemms(n, st)
            sh = None
            if cfg.shared_I:
                mark("shared")
                sh = shared[:n]
                moe.moe_grouped_gemm1_act(xd[sl], off_s[n], WS1, cfg.shared_I, hs[:n], stream=st,
                                          split=False, **act_kw)
                moe.moe_grouped_gemm2(hs[:n], off_s[n], WS2, H, sh, stream=st, split=False)
            mark(fin_stage)
            wf = None if w_in else wts[sl]
            if args.fused_tail:
                moe.moe_finalize_add_rmsnorm(y, wf, pmap[sl], residual[sl], gamma, 1e-6, 1.0, sh,
                                             out[sl], stream=st)
            else:
                moe.moe_finalize(y, wf, pmap[sl], 1.0, sh, out[sl], stream=st)
        mark(None)

    marks_per_step = len(chunks) * len(stages) + 1

    # Steps of a few dozen microseconds (decode batches, the tiny layer) are
    # timed from their events with a GPU spin before each (outside the
    # events) that keeps the GPU busy while the host enqueues the step, so
    # the events time the kernels, not the Python call overhead between them.
    host_ahead = decode or T * k <= 256

    def step(i, ev=None):
        if flush is not None:
            evict_caches()
        if host_ahead:
            torch.cuda._sleep(HOST_AHEAD_CYCLES)
        if ev is None:
            layer(i % len(dev_draws), stream)
            return
        names, pool = ev
        it = iter(pool)

        def mark(name):
            names.append(name)
            next(it).record(stream)
        layer(i % len(dev_draws), stream, mark)

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    graphs = []
    if args.graph:
        # one graph per input batch; the cache eviction stays outside the graph
        for d in range(len(dev_draws)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                layer(d, torch.cuda.current_stream())
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
    # Timed pass 1, the throughput: whole steps, one event pair around each
    # (an event between two kernels of one stream still leaves the GPU idle a
    # few microseconds on this runtime, so the stage events of pass 2 would
    # inflate short steps)
    step_ev = [(TimingEvent(), TimingEvent()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if flush is not None:
            evict_caches()
        if host_ahead:
            torch.cuda._sleep(HOST_AHEAD_CYCLES)  # the step is enqueued meanwhile
        step_ev[i][0].record()
        if graphs:
            graphs[i % len(graphs)].replay()
        else:
            layer(i % len(dev_draws), stream)
        step_ev[i][1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = np.array([a.elapsed_time(b) for a, b in step_ev])

    # Timed pass 2, the breakdown: the same steps with an event before every
    # stage (not under graph replay)
    stage_steps = args.steps if graphs else min(args.steps, 100)
    events = [([], [TimingEvent() for _ in range(marks_per_step)]) for _ in range(stage_steps)]
    if not graphs:
        torch.cuda.synchronize()
        for i in range(stage_steps):
            step(i, events[i])
        torch.cuda.synchronize()

    # per step: milliseconds of each stage, summed over the step's chunks
    per_step = []
    for i in range(stage_steps):
        if graphs:
            per_step.append({"layer_graph": float(step_ms[i])})
            continue
        names, pool = events[i]
        ms = dict.fromkeys(stages, 0.0)
        for j in range(len(names) - 1):
            ms[names[j]] += pool[j].elapsed_time(pool[j + 1])
        per_step.append(ms)
    stage_ms = {s: float(np.mean([p[s] for p in per_step])) for s in per_step[0]}

    # routed rows per local expert of every chunk of every draw (untimed
    # re-run of route + permute)
    draw_counts = []
    for d in range(len(dev_draws)):
        per_chunk = []
        for t0, n in chunks:
            route_permute(d, t0, n)
            per_chunk.append(chunk_counts())
        draw_counts.append(per_chunk)

    # algorithmic work of every timed step (throughput) and of the per-stage
    # pass's steps (the GEMM1 roofline)
    work = [[(gemm_work(cfg, c, 1), gemm_work(cfg, c, 2)) for c in per_chunk]
            for per_chunk in draw_counts]
    flops_step = [6.0 * T * H * cfg.shared_I
                  + sum(f1 + f2 for (f1, _), (f2, _) in work[i % len(dev_draws)])
                  for i in range(args.steps)]
    g1_flops = g1_bytes = g1_ms = g2_bytes = 0.0
    for i in range(stage_steps):
        for (f1, b1), (f2, b2) in work[i % len(dev_draws)]:
            g1_flops += f1
            g1_bytes += b1
            g2_bytes += b2
        # (with the fused first stage its time, routing included, stands for GEMM1)
        g1_ms += per_step[i].get("gemm1", per_step[i].get("route_permute_gemm1", 0.0))
    if host_ahead:
        # the flush and the spin between steps are not part of the layer:
        # time from the events around each step
        ms_per_step = float(np.mean(step_ms))
    else:
        ms_per_step = elapsed / args.steps * 1e3
    # the same steps with an event before every stage
    ms_per_step_staged = float(np.mean([sum(p.values()) for p in per_step]))
    tflops = float(np.mean(flops_step)) / (ms_per_step * 1e-3) / 1e12
    g1_s = g1_ms * 1e-3 if g1_ms > 0 else float("nan")  # no per-kernel events under graph replay
    # (two-term rows run the fp8 MFMA twice: the bf16 peak is their rate)
    peak_mfma = PEAK_FP8_TFLOPS if (cfg.fp8 or cfg.fp8_block) else PEAK_BF16_TFLOPS
    t_mfma = g1_flops / (peak_mfma * 1e12)
    t_hbm = g1_bytes / (PEAK_HBM_GBS * 1e9)
    if t_mfma >= t_hbm:
        achieved = g1_flops / g1_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak_mfma,
                "unit": "TFLOP/s", "frac": achieved / peak_mfma}
    else:
        achieved = g1_bytes / g1_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    n_launch = stage_steps * len(chunks)
    if graphs:
        roof.update({"achieved": None, "frac": None,
                     "note": "no per-kernel timing under graph replay; run without --graph"})
    roof.update({"traffic": measured_traffic(label),
                 "kernel": ("route_permute_gemm1_act (router, permute map and GEMM1 in one launch;"
                            " its time includes the routing)" if fused_g1 else "grouped_gemm1_act"),
                 "algorithmic_flop_per_launch": g1_flops / n_launch,
                 "algorithmic_bytes_per_launch": g1_bytes / n_launch,
                 "gemm2_algorithmic_bytes_per_launch": g2_bytes / n_launch})

    counts0 = np.sum(draw_counts[0], axis=0)
    result = {
        "metric": METRIC,
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_staged": ms_per_step_staged,
        "stage_steps": stage_steps,
        "ms_per_step_median": float(np.median(step_ms)),
        "ms_per_step_min": float(np.min(step_ms)),
        "ms_per_step_max": float(np.max(step_ms)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8 (blockwise: 128-element activation groups, 128 x 128 weight blocks)"
                  if cfg.fp8_block else "fp8" if cfg.fp8
                  else "fp8x2 (two E4M3 terms) x e2m1" if cfg.fp8x2 else "bf16"),
        "data": "synthetic (seeded N(0,1) activations, N(0,1/sqrt(fan_in)) random weights"
                + (", MXFP4-quantized" if cfg.mxfp4 else "")
                + ((", FP8 E4M3 activations per token" if cfg.mxfp4 else
                    ", FP8 E4M3 weights per channel, activations per token") if cfg.fp8 else "")
                + (", bf16 activations as two FP8 E4M3 terms per token" if cfg.fp8x2 else "")
                + (", FP8 E4M3 weights per 128 x 128 block, activations per token and 128-element"
                   " group" if cfg.fp8_block else "")
                + ")",
        "config": {"workload": label, "tokens": T, "hidden": H, "intermediate": I,
                   "experts": E, "local_experts": El, "top_k": k,
                   "shared_intermediate": cfg.shared_I,
                   "expert_weights": "mxfp4 (e2m1 + E8M0 per 32)" if cfg.mxfp4 else
                                     ("fp8 e4m3 (fp32 scale per 128 x 128 block)" if cfg.fp8_block
                                      else "fp8 e4m3 (fp32 scale per channel)" if cfg.fp8
                                      else "bf16"),
                   "routing": ("softmax" if cfg.score == 0 else "sigmoid") +
                              (f" top-{k} renormalized") + (f", rsf {cfg.rsf}" if cfg.rsf != 1 else "") +
                              (f", Zipf({cfg.zipf_s}) logit bias" if cfg.zipf_s else ""),
                   "form": (("deferred + separate finalize, L2/MALL evicted (512 MiB read) before each step, "
                             f"{len(draws)} routing draws" if decode else "finalized")
                            + (", the host enqueues each step while a GPU spin runs ahead of it "
                               "(events time the kernels, not the Python call overhead)"
                               if host_ahead else ""))
                           + (", replayed as a captured HIP graph" if graphs else "")
                           + (", fused tail (finalize + residual add + RMSNorm)" if args.fused_tail else "")
                           + (f", {len(chunks)} chunks of {P} tokens" if len(chunks) > 1 else "")
                           + (f", batched experts format ({Mb} rows per expert)" if Mb else "")
                           + (", rows gathered through the inverse map inside GEMM1"
                              if gathered or gathered_q else ""),
                   "activation": args.activation
                                 + (f", clamp {args.activation_clamp:g}" if args.activation_clamp else "")
                                 + (", routing weight on the input" if w_in else "")},
        "tflops": tflops,
        "mfma_frac_layer": tflops / peak_mfma,
        "stages_ms": stage_ms,
        "expert_rows": counts0.tolist() if len(counts0) <= 16 else
                       {"min": int(counts0.min()), "max": int(counts0.max()),
                        "mean": float(counts0.mean()), "touched": int((counts0 > 0).sum())},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        del dev_draws, W1, W2, x_perm, h, y, out
        result["cpu_baseline"] = cpu_baseline(cfg, draws, w, args.cpu_seconds, variant)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
