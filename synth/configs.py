"""The five fused-MoE workloads and their seeded input recipes.

Sizes, routing functions and distributions are those of the workload
descriptions: a tiny layer, a Mixtral-8x7B-shaped prefill, a DeepSeek-V3-shaped
routed layer with a shared expert, one expert-parallel rank's share at decode
batch sizes, and the DeepSeek-V3 shape with MXFP4 expert weights.  Weights are
random (no trained checkpoints): N(0, 1/sqrt(fan_in)) rounded to bf16.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

from . import (TID_LOGITS, TID_W1, TID_W2, TID_WS1, TID_WS2, TID_X, biased_logits,
               fp8_quantize_blocks, fp8_quantize_rows, mxfp4_quantize, normal_bf16, normal_f32,
               zipf_log_bias)

SOFTMAX, SIGMOID = 0, 1


@dataclasses.dataclass(frozen=True)
class MoeConfig:
    name: str
    T: int                 # tokens
    H: int                 # hidden
    I: int                 # expert intermediate
    E: int                 # global experts
    k: int                 # top_k
    score: int             # SOFTMAX or SIGMOID
    renormalize: bool
    rsf: float             # routed scaling factor folded into the weights
    seed: int
    E_local: Optional[int] = None   # None: all experts local
    local_first: int = 0            # first global id owned by this rank
    shared_I: int = 0               # shared-expert intermediate (0: none)
    mxfp4: bool = False
    fp8: bool = False               # FP8 E4M3 activations (per token); weights FP8 per channel
                                    # unless mxfp4
    fp8x2: bool = False             # bf16 activations carried as two FP8 E4M3 terms
                                    # (MXFP4 weights)
    fp8_block: bool = False         # blockwise FP8: activations per 128-element group,
                                    # weights per 128 x 128 block
    zipf_s: float = 0.0             # Zipf exponent of the logit bias (0: none)
    deferred: bool = False

    @property
    def El(self) -> int:
        return self.E if self.E_local is None else self.E_local

    def with_T(self, T: int) -> "MoeConfig":
        return dataclasses.replace(self, T=T)


TINY = MoeConfig("tiny_16tok_h128_i256_e8_k2", T=16, H=128, I=256, E=8, k=2,
                 score=SOFTMAX, renormalize=True, rsf=1.0, seed=1)
MIXTRAL = MoeConfig("mixtral8x7b_prefill_4096tok", T=4096, H=4096, I=14336, E=8, k=2,
                    score=SOFTMAX, renormalize=True, rsf=1.0, seed=2, zipf_s=1.1)
DEEPSEEK = MoeConfig("deepseekv3_routed_shared_2048tok", T=2048, H=7168, I=2048, E=256, k=8,
                     score=SIGMOID, renormalize=True, rsf=2.5, seed=3, shared_I=2048)
EP_DECODE = MoeConfig("ep_rank3of8_decode", T=64, H=7168, I=2048, E=256, k=8,
                      score=SIGMOID, renormalize=True, rsf=2.5, seed=4, E_local=32,
                      local_first=96, deferred=True)
DEEPSEEK_MXFP4 = MoeConfig("deepseekv3_mxfp4_2048tok", T=2048, H=7168, I=2048, E=256, k=8,
                           score=SIGMOID, renormalize=True, rsf=2.5, seed=5, mxfp4=True)

# FP8 variants of the two prefill shapes: weights quantized per output channel
# from the same bf16 draws, activations quantized per token inside the layer
MIXTRAL_FP8 = MoeConfig("mixtral8x7b_fp8_prefill_4096tok", T=4096, H=4096, I=14336, E=8, k=2,
                        score=SOFTMAX, renormalize=True, rsf=1.0, seed=2, zipf_s=1.1, fp8=True)
DEEPSEEK_FP8 = MoeConfig("deepseekv3_fp8_2048tok", T=2048, H=7168, I=2048, E=256, k=8,
                         score=SIGMOID, renormalize=True, rsf=2.5, seed=3, fp8=True)

# MXFP4 weights with FP8 activations: FP8 x e2m1 on the matrix cores
DEEPSEEK_MXFP4_FP8 = MoeConfig("deepseekv3_mxfp4_fp8act_2048tok", T=2048, H=7168, I=2048, E=256,
                               k=8, score=SIGMOID, renormalize=True, rsf=2.5, seed=5, mxfp4=True,
                               fp8=True)

# the MXFP4 workload with its bf16 activations carried to the FP8 x e2m1
# matrix cores as two FP8 terms per token (and per hidden row)
DEEPSEEK_MXFP4_X2 = MoeConfig("deepseekv3_mxfp4_x2act_2048tok", T=2048, H=7168, I=2048, E=256,
                              k=8, score=SIGMOID, renormalize=True, rsf=2.5, seed=5, mxfp4=True,
                              fp8x2=True)

# blockwise FP8 (128 x 128 weight blocks, 128-element activation groups, as
# DeepSeek-V3 stores its weights) on the DeepSeek-V3 routed shape
DEEPSEEK_FP8_BLOCK = MoeConfig("deepseekv3_fp8block_2048tok", T=2048, H=7168, I=2048, E=256, k=8,
                               score=SIGMOID, renormalize=True, rsf=2.5, seed=3, fp8_block=True)

ALL = {c.name: c for c in (TINY, MIXTRAL, DEEPSEEK, EP_DECODE, DEEPSEEK_MXFP4, MIXTRAL_FP8,
                           DEEPSEEK_FP8, DEEPSEEK_MXFP4_FP8, DEEPSEEK_MXFP4_X2,
                           DEEPSEEK_FP8_BLOCK)}

EP_DECODE_BATCHES = (1, 8, 64)
EP_DECODE_DRAWS = 16
EP_DECODE_DRAW_SEED0 = 400


def expert_map(cfg: MoeConfig) -> Optional[np.ndarray]:
    """Global expert id -> local id (or -1), int32 [E]; None when all are local."""
    if cfg.E_local is None:
        return None
    m = np.full(cfg.E, -1, dtype=np.int32)
    m[cfg.local_first:cfg.local_first + cfg.E_local] = np.arange(cfg.E_local, dtype=np.int32)
    return m


def make_activations(cfg: MoeConfig, seed: Optional[int] = None):
    """x bf16 bits [T, H] ~ N(0,1); logits fp32 [T, E] ~ N(0,1) (+ ln p_e when Zipf-biased)."""
    s = cfg.seed if seed is None else seed
    x = normal_bf16(s, TID_X, (cfg.T, cfg.H))
    if cfg.zipf_s:
        logits = biased_logits(s, TID_LOGITS, cfg.T, zipf_log_bias(cfg.E, cfg.zipf_s))
    else:
        logits = normal_f32(s, TID_LOGITS, (cfg.T, cfg.E))
    return x, logits


def make_weights(cfg: MoeConfig):
    """Local expert weights: w1 [E_l, 2I, H], w2 [E_l, H, I] bf16 bits, std 1/sqrt(fan_in).

    Returns a dict; MXFP4 configs also carry the packed bytes and E8M0 scales
    (w1_q/w1_s, w2_q/w2_s) quantized from the same bf16 draw."""
    El, H, I = cfg.El, cfg.H, cfg.I
    w = {
        "w1": normal_bf16(cfg.seed, TID_W1, (El, 2 * I, H), std=1.0 / math.sqrt(H)),
        "w2": normal_bf16(cfg.seed, TID_W2, (El, H, I), std=1.0 / math.sqrt(I)),
    }
    if cfg.shared_I:
        Is = cfg.shared_I
        w["ws1"] = normal_bf16(cfg.seed, TID_WS1, (2 * Is, H), std=1.0 / math.sqrt(H))
        w["ws2"] = normal_bf16(cfg.seed, TID_WS2, (H, Is), std=1.0 / math.sqrt(Is))
    if cfg.mxfp4:
        w["w1_q"], w["w1_s"] = mxfp4_quantize(w["w1"])
        w["w2_q"], w["w2_s"] = mxfp4_quantize(w["w2"])
        del w["w1"], w["w2"]
    elif cfg.fp8_block:
        w["w1_q"], w["w1_s"] = fp8_quantize_blocks(w["w1"])
        w["w2_q"], w["w2_s"] = fp8_quantize_blocks(w["w2"])
        del w["w1"], w["w2"]
    elif cfg.fp8:
        w["w1_q"], w["w1_s"] = fp8_quantize_rows(w["w1"])
        w["w2_q"], w["w2_s"] = fp8_quantize_rows(w["w2"])
        del w["w1"], w["w2"]
    return w


def permuted_rows(T: int, k: int) -> int:
    """Padded permuted row count used by the tests and bench: round_up(T*k, 128)."""
    return ((T * k + 127) // 128) * 128
