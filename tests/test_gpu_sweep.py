"""Seeded random whole layers against the oracle.

Forty small layers whose expert count, top-k, token count, widths, expert
map (all experts local, or a scattered subset), scoring, renormalisation,
routed scaling factor, logit ties, shared expert and weight format (bf16 or
MXFP4) are drawn from a seeded generator, so that the tile shapes, the
decode kernels, the split and tail reductions and the one-launch router
paths meet shapes nobody picked by hand.  Each layer runs through the fused
entry point and is checked against the oracle's per-token mixture: the
router's ids bit-exact, every token's output within the bar (1e-2 relative
Frobenius for bf16 weights, 3e-2 for MXFP4), tokens with nothing to add
exactly zero.  The deferred form of the same layer gives the same map as the
permute call, and its separate finalize the same output within rounding.

Forty more layers draw the quantized formats and the layer options on top:
FP8 weights with per-row activations (dynamic or static scales), block-scaled
FP8 with per-group activations, MXFP4 weights with one- or two-term FP8
activations, bf16; GELU or SiLU, a clamp, the routing weight on the input
(top-1), chunked passes and the batched experts layout.  The oracle sees the
same options and quantizes from its own bf16 rounding of the hidden rows, so a
hidden element's code can differ from the kernels' by one E4M3 step where the
two bf16 roundings fall on either side of a rounding midpoint.  One step is
1/16 to 1/8 of the element; for a large element of a top-1 token that is a
few percent of the token (seen: an element near 4.55 with a static scale of
0.03, one step = 3.2 % of its token).  So the per-token bar for FP8
activations is 6e-2, and the pooled bar stays 1e-2 (3e-2 with MXFP4 weights).

Thirteen fixed layers add the limits and the degenerate shapes: 1024 experts
with top-32 (decode- and prefill-sized, all local or a scattered subset, bf16,
MXFP4, FP8, blockwise FP8, two-term, batched), k = E, a single expert, a
single local expert of 256, whose tokens mostly have nothing to add, and FP8
decode batches with static scales, the router weight on the input and the
batched layout.
"""
import gc

import numpy as np
import pytest
import torch

import mixture_experts_layer_scan_amd as moe
import oracle
import synth

from gpu_util import (dev, dev_bf16, host_f64, need_gpu, per_row_rel, rel_fro,
                      sample_tokens)

pytestmark = pytest.mark.gpu

N_LAYERS = 40


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _draw(i: int) -> dict:
    rng = np.random.default_rng(9000 + i)
    E = int(rng.choice([4, 8, 16, 32, 64, 128, 256]))
    c = {
        "seed": 9000 + i,
        "E": E,
        "k": int(rng.integers(1, min(8, E) + 1)),
        "T": int(rng.choice([1, 2, 3, 5, 8, 13, 16, 17, 31, 64, 65, 127, 200, 333, 512, 777, 1024,
                             1500])),
        "H": int(rng.choice([128, 256, 384, 512, 768])),
        "I": int(rng.choice([64, 128, 192, 256, 320, 512])),
        "mxfp4": bool(rng.random() < 0.25),
        "score": int(rng.integers(0, 2)),
        "renormalize": bool(rng.random() < 0.8),
        "rsf": float(rng.choice([1.0, 2.5])),
        "ties": bool(rng.random() < 0.2),
        "shared_I": int(rng.choice([64, 128, 256])) if rng.random() < 0.25 else 0,
    }
    if rng.random() < 0.4:
        El = int(rng.integers(1, E + 1))
        emap = np.full(E, -1, dtype=np.int32)
        emap[rng.choice(E, size=El, replace=False)] = np.arange(El, dtype=np.int32)
        c["El"], c["emap"] = El, emap
    else:
        c["El"], c["emap"] = E, None
    return c


def _name(c: dict) -> str:
    return (f"T{c['T']}_E{c['E']}l{c['El']}_k{c['k']}_H{c['H']}_I{c['I']}"
            f"{'_mxfp4' if c['mxfp4'] else ''}{'_sig' if c['score'] else ''}"
            f"{'' if c['renormalize'] else '_raw'}{'_ties' if c['ties'] else ''}"
            f"{'_sh' + str(c['shared_I']) if c['shared_I'] else ''}")


def _fixed(seed, T, E, k, H, I, El=None, mxfp4=False, score=0, shared_I=0):
    c = {"seed": seed, "E": E, "k": k, "T": T, "H": H, "I": I, "mxfp4": mxfp4, "score": score,
         "renormalize": True, "rsf": 2.5 if score else 1.0, "ties": False, "shared_I": shared_I,
         "El": E, "emap": None}
    if El is not None:
        emap = np.full(E, -1, dtype=np.int32)
        emap[np.random.default_rng(seed).choice(E, size=El, replace=False)] = np.arange(El)
        c["El"], c["emap"] = El, emap
    return c


# the limits and degenerate shapes: 1024 experts with top-32 (decode-sized
# and prefill-sized, all local and a scattered tenth), k = E, one expert, one
# local expert of many
EXTREME = [
    _fixed(9900, 2, 1024, 32, 128, 64),
    _fixed(9901, 300, 1024, 32, 256, 128, El=100, score=1),
    _fixed(9902, 64, 1024, 32, 128, 64, mxfp4=True),
    _fixed(9903, 37, 4, 4, 256, 128),
    _fixed(9904, 33, 1, 1, 128, 64, shared_I=64),
    _fixed(9905, 200, 256, 8, 256, 128, El=1, score=1),
]

CASES = [_draw(i) for i in range(N_LAYERS)] + EXTREME


@pytest.mark.parametrize("c", CASES, ids=[_name(c) for c in CASES])
def test_random_layer(c):
    s, T, E, El, k, H, I, Is = (c["seed"], c["T"], c["E"], c["El"], c["k"], c["H"], c["I"],
                                c["shared_I"])
    x = synth.normal_bf16(s, 0, (T, H))
    logits = synth.normal_f32(s, 1, (T, E))
    if c["ties"]:
        logits = (np.round(logits * 4.0) / 4.0).astype(np.float32)  # many equal logits
    w1 = synth.normal_bf16(s, 2, (El, 2 * I, H), std=1 / np.sqrt(H))
    w2 = synth.normal_bf16(s, 3, (El, H, I), std=1 / np.sqrt(I))
    if c["mxfp4"]:
        q1, s1 = synth.mxfp4_quantize(w1)
        q2, s2 = synth.mxfp4_quantize(w2)
        W1, W2 = moe.Weights(dev(q1), dev(s1)), moe.Weights(dev(q2), dev(s2))
        O1, O2 = oracle.Weights(q1, s1), oracle.Weights(q2, s2)
    else:
        W1, W2 = moe.Weights(dev_bf16(w1)), moe.Weights(dev_bf16(w2))
        O1, O2 = oracle.Weights(w1), oracle.Weights(w2)
    ws1 = ws2 = None
    if Is:
        ws1 = synth.normal_bf16(s, 4, (2 * Is, H), std=1 / np.sqrt(H))
        ws2 = synth.normal_bf16(s, 5, (H, Is), std=1 / np.sqrt(Is))
    ref = oracle.moe_tokens(x, logits, O1, O2, I, k, c["score"], c["renormalize"], c["rsf"],
                            expert_map=c["emap"], shared_I=Is, ws1=ws1, ws2=ws2)

    ld, xd = dev(logits), dev_bf16(x)
    emap_d = None if c["emap"] is None else dev(c["emap"])
    sh = {} if not Is else {"ws1": dev_bf16(ws1), "ws2": dev_bf16(ws2)}
    out = moe.moe_fused_experts(ld, xd, W1, W2, k, c["score"], c["renormalize"], c["rsf"],
                                expert_map=emap_d, **sh)
    ids, _ = moe.moe_route_topk(ld, k, c["score"], c["renormalize"], c["rsf"])
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])

    bar = 3e-2 if c["mxfp4"] else 1e-2
    got = host_f64(out)
    per_tok = per_row_rel(got, ref["out"])
    assert per_tok.max() < bar, (int(per_tok.argmax()), float(per_tok.max()))
    assert rel_fro(got, ref["out"]) < bar

    if Is:
        return  # the deferred form carries no shared expert
    # deferred: the same map as the permute call, and its finalize the same output
    y_perm, w_bf16, pmap = moe.moe_fused_experts_unfinalized(
        ld, xd, W1, W2, k, c["score"], c["renormalize"], c["rsf"], expert_map=emap_d)
    p = moe.moe_permute(ids, E, El, emap_d, xd)
    fin = moe.moe_finalize(y_perm, w_bf16, pmap)
    torch.cuda.synchronize()
    assert np.array_equal(pmap.cpu().numpy(), p["map"].cpu().numpy())
    assert rel_fro(host_f64(fin), got) < 1e-2


def _draw_variant(i: int) -> dict:
    rng = np.random.default_rng(9500 + i)
    fmt = str(rng.choice(["fp8", "block", "w4a8", "x2", "bf16"], p=[0.25, 0.2, 0.15, 0.2, 0.2]))
    q = {"w4a8": 256, "x2": 256, "fp8": 128, "block": 128, "bf16": 64}[fmt]
    E = int(rng.choice([4, 8, 16, 32, 64, 128]))
    k = int(rng.integers(1, min(8, E) + 1))
    T = int(rng.choice([1, 2, 4, 7, 16, 33, 64, 100, 257, 640, 1024]))
    c = {
        "seed": 9500 + i, "fmt": fmt, "E": E, "k": k, "T": T,
        "H": q * int(rng.integers(1, 1024 // q + 1)),
        "I": q * int(rng.integers(1, 512 // q + 1)),
        "score": int(rng.integers(0, 2)),
        "renormalize": bool(rng.random() < 0.7),
        "rsf": float(rng.choice([1.0, 2.5])),
        "act": str(rng.choice(["silu", "gelu"])),
        "clamp": float(rng.choice([0.0, 0.0, 0.75, 7.0])),
        "shared_I": int(rng.choice([64, 128, 256])) if rng.random() < 0.2 else 0,
        "chunk": int(rng.integers(1, T)) if T > 1 and rng.random() < 0.25 else 0,
        "batched": bool(rng.random() < 0.2),
        "on_input": bool(k == 1 and fmt != "block" and rng.random() < 0.6),
        "static": bool(fmt in ("fp8", "w4a8") and rng.random() < 0.3),
    }
    if rng.random() < 0.4:
        El = int(rng.integers(1, E + 1))
        emap = np.full(E, -1, dtype=np.int32)
        emap[rng.choice(E, size=El, replace=False)] = np.arange(El, dtype=np.int32)
        c["El"], c["emap"] = El, emap
    else:
        c["El"], c["emap"] = E, None
    return c


def _vname(c: dict) -> str:
    return (f"{c['fmt']}_T{c['T']}_E{c['E']}l{c['El']}_k{c['k']}_H{c['H']}_I{c['I']}"
            f"_{c['act']}{'_c' + str(c['clamp']) if c['clamp'] else ''}"
            f"{'_sig' if c['score'] else ''}{'' if c['renormalize'] else '_raw'}"
            f"{'_sh' + str(c['shared_I']) if c['shared_I'] else ''}"
            f"{'_ch' + str(c['chunk']) if c['chunk'] else ''}{'_bat' if c['batched'] else ''}"
            f"{'_oninput' if c['on_input'] else ''}{'_static' if c['static'] else ''}")


def _vfixed(seed, fmt, T, E, k, H, I, El=None, **opt):
    c = _fixed(seed, T, E, k, H, I, El=El, score=1)
    c.update(fmt=fmt, act="silu", clamp=0.0, chunk=0, batched=False, on_input=False,
             static=False)
    c.update(opt)
    return c


# the quantized formats at the routing limits, and the batched layout with
# top-32 over a scattered map
VEXTREME = [
    _vfixed(9950, "fp8", 64, 1024, 32, 256, 128),
    _vfixed(9951, "block", 300, 512, 16, 256, 256, El=64),
    _vfixed(9952, "x2", 2, 1024, 32, 256, 256),
    _vfixed(9953, "bf16", 100, 1024, 32, 128, 64, El=200, batched=True, act="gelu"),
    # the whole-k FP8 decode GEMMs under the layer options: static scales
    # with GELU and a clamp, the router weight on the input, the batched layout
    _vfixed(9954, "fp8", 3, 64, 4, 1024, 512, El=40, static=True, act="gelu", clamp=7.0),
    _vfixed(9955, "fp8", 5, 16, 1, 1024, 512, on_input=True),
    _vfixed(9956, "fp8", 6, 32, 8, 2048, 1024, batched=True),
]

VCASES = [_draw_variant(i) for i in range(N_LAYERS)] + VEXTREME
# the oracle checks a spread of tokens (first and last included) of the large layers
ORACLE_TOKENS = 192


def _weights(c, s, w1, w2):
    """(device W1, W2, oracle W1, W2, fp8 option) for the drawn format."""
    fmt = c["fmt"]
    if fmt in ("w4a8", "x2"):
        (q1, s1), (q2, s2) = synth.mxfp4_quantize(w1), synth.mxfp4_quantize(w2)
        return (moe.Weights(dev(q1), dev(s1)), moe.Weights(dev(q2), dev(s2)),
                oracle.Weights(q1, s1), oracle.Weights(q2, s2), "x2" if fmt == "x2" else True)
    if fmt == "fp8":
        (q1, s1), (q2, s2) = synth.fp8_quantize_rows(w1), synth.fp8_quantize_rows(w2)
        return (moe.Weights(dev(q1), dev(s1)), moe.Weights(dev(q2), dev(s2)),
                oracle.Weights(q1, s1.reshape(-1)), oracle.Weights(q2, s2.reshape(-1)), True)
    if fmt == "block":
        (q1, s1), (q2, s2) = synth.fp8_quantize_blocks(w1), synth.fp8_quantize_blocks(w2)
        return (moe.Weights(dev(q1), dev(s1)), moe.Weights(dev(q2), dev(s2)),
                oracle.Weights(q1, s1, block=True), oracle.Weights(q2, s2, block=True), "block")
    return (moe.Weights(dev_bf16(w1)), moe.Weights(dev_bf16(w2)),
            oracle.Weights(w1), oracle.Weights(w2), False)


@pytest.mark.parametrize("c", VCASES, ids=[_vname(c) for c in VCASES])
def test_random_variant_layer(c):
    s, T, E, El, k, H, I, Is = (c["seed"], c["T"], c["E"], c["El"], c["k"], c["H"], c["I"],
                                c["shared_I"])
    x = synth.normal_bf16(s, 0, (T, H))
    logits = synth.normal_f32(s, 1, (T, E))
    w1 = synth.normal_bf16(s, 2, (El, 2 * I, H), std=1 / np.sqrt(H))
    w2 = synth.normal_bf16(s, 3, (El, H, I), std=1 / np.sqrt(I))
    W1, W2, O1, O2, fp8 = _weights(c, s, w1, w2)
    ws1 = ws2 = None
    if Is:
        ws1 = synth.normal_bf16(s, 4, (2 * Is, H), std=1 / np.sqrt(H))
        ws2 = synth.normal_bf16(s, 5, (H, Is), std=1 / np.sqrt(Is))
    # static scales: the tokens' largest magnitude over the E4M3 range, and a
    # fixed one for the hidden rows (their largest values near 10 here; the
    # few beyond 448 * a2 saturate on both sides alike)
    a1 = a2 = None
    if c["static"]:
        a1 = float(np.abs(synth.bf16_bits_to_f32(x)).max() / np.float32(448.0))
        a2 = 0.03
    toks = (sample_tokens(T, ORACLE_TOKENS, s) if T * k > 2048 else None)
    ref = oracle.moe_tokens(x, logits, O1, O2, I, k, c["score"], c["renormalize"], c["rsf"],
                            expert_map=c["emap"], shared_I=Is, ws1=ws1, ws2=ws2, tokens=toks,
                            activation=c["act"], clamp=c["clamp"], weight_on_input=c["on_input"],
                            fp8=fp8, a1_scale=a1, a2_scale=a2)

    ld, xd = dev(logits), dev_bf16(x)
    emap_d = None if c["emap"] is None else dev(c["emap"])
    sh = {} if not Is else {"ws1": dev_bf16(ws1), "ws2": dev_bf16(ws2)}
    opts = dict(expert_map=emap_d, activation=c["act"], activation_clamp=c["clamp"],
                apply_router_weight_on_input=c["on_input"], fp8=fp8,
                batched_max_tokens=T if c["batched"] else 0)
    if c["static"]:
        opts.update(a1_scale=torch.tensor([a1], device="cuda"),
                    a2_scale=torch.tensor([a2], device="cuda"))
    out = moe.moe_fused_experts(ld, xd, W1, W2, k, c["score"], c["renormalize"], c["rsf"],
                                chunk_tokens=c["chunk"], **sh, **opts)
    torch.cuda.synchronize()

    got = host_f64(out, toks)
    tok_bar = 6e-2 if fp8 else 1e-2
    pool_bar = 3e-2 if c["fmt"] in ("w4a8", "x2") else 1e-2
    per_tok = per_row_rel(got, ref["out"])
    assert per_tok.max() < tok_bar, (int(per_tok.argmax()), float(per_tok.max()))
    assert rel_fro(got, ref["out"]) < pool_bar

    if Is:
        return  # the deferred form carries no shared expert
    # deferred, one pass: its finalize gives the fused output within rounding
    y_perm, w_bf16, pmap = moe.moe_fused_experts_unfinalized(
        ld, xd, W1, W2, k, c["score"], c["renormalize"], c["rsf"], **opts)
    fin = moe.moe_finalize(y_perm, w_bf16, pmap)
    torch.cuda.synchronize()
    assert rel_fro(host_f64(fin), host_f64(out)) < 1e-2
