"""The whole routed-expert MoE layer, chained from the oracle's steps.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Order of the steps ([ATOM] "Stage D: MXFP4 Fused MoE" and "Stage B: Dynamic
Activation Quantization"; [NVFP4] "Weight Dequantization and Activation QDQ"):
route -> permute -> (activation quantization) -> stage 1 (gate/up, SiLU*up)
-> (activation quantization of h) -> stage 2 (down) -> combine.

Activation paths:
  bf16   activations enter the GEMM as bf16 (weights dequantized in the tile)
  mx     activations are quantized with mxfp4_quant_1x32 before each GEMM
  nvfp4  activations pass the NVFP4 QDQ round trip before each GEMM
  fp8    activations are quantized to FP8 E4M3 per row (per token before
         stage 1, per sorted row of h before stage 2) before each GEMM

`weights` maps names to per-expert indexable arrays:
  w13, w13_scale, w2, w2_scale and, for nvfp4, w13_ts / w2_ts (float32 [E]).
Only experts that receive rows are read.
"""

import numpy as np

from . import formats as F
from . import route as R
from . import permute as P
from . import quant as Q
from . import gemm as G


def activation_values(afmt, x_bits):
    """The float64 values a GEMM sees for bf16 activations x_bits [M, K]."""
    if afmt == "bf16":
        return F.bf16_decode(x_bits)
    if afmt == "mx":
        return Q.mxfp4_qdq_values(x_bits)
    if afmt == "nvfp4":
        if x_bits.shape[0] == 0:
            return np.zeros(x_bits.shape)
        return F.bf16_decode(Q.nvfp4_qdq(x_bits)["y"])
    if afmt == "fp8":
        return Q.fp8_qdq_values(x_bits)
    raise ValueError(afmt)


def stage2_activation(afmt, h, h_bits, rounding=True):
    """The values stage 2 sees for the stage-1 output of the sorted rows.

    h is rounded to bf16 (h_bits) and then takes the same activation path as x
    ([ATOM] "Stage B: Dynamic Activation Quantization": each GEMM's live
    activations are quantized at run time; [NVFP4] "Weight Dequantization and
    Activation QDQ": a QDQ round trip before each GEMM).  For NVFP4 the
    dynamic tensor scale is taken over all sorted rows [0, n_rows) of h at
    once, as over all tokens of x before stage 1.  With rounding off the
    unrounded h passes straight through.
    """
    if not rounding:
        return h
    return activation_values(afmt, h_bits)


def weight_getter(wfmt, weights, name):
    def get(e):
        if wfmt == "nvfp4":
            return G.dequant_expert(wfmt, weights[name][e], weights[name + "_scale"][e],
                                    weights[name + "_ts"][e])
        return G.dequant_expert(wfmt, weights[name][e], weights[name + "_scale"][e])
    return get


def moe_layer(x_bits, logits, bias, weights, *, E, n_shared, n_group, topk_group, topk,
              afmt, wfmt, block_m=16, renormalize=True, routed_scale=1.0, rounding=True,
              topk_ids=None, topk_w=None):
    """Run the layer.  Returns a dict with every intermediate result."""
    T = x_bits.shape[0]
    if topk_ids is None:
        topk_ids, topk_w = R.moe_route(logits, bias, n_group, topk_group, topk,
                                       renormalize, routed_scale)
    perm = P.moe_permute(topk_ids, E, n_shared, block_m)
    k = topk + n_shared
    n_rows = int(perm["expert_offsets"][-1])
    tok = perm["sorted_pairs"][:n_rows] // k
    a1 = activation_values(afmt, x_bits)[tok]
    h = G.grouped_stage(1, a1, perm["expert_offsets"], weight_getter(wfmt, weights, "w13"),
                        rounding)
    h_bits = F.bf16_bits(h)
    a2 = stage2_activation(afmt, h, h_bits, rounding)
    y = G.grouped_stage(2, a2, perm["expert_offsets"], weight_getter(wfmt, weights, "w2"),
                        rounding)
    y_bits = F.bf16_bits(y)
    out, out_bits = G.moe_combine(y if not rounding else F.bf16_decode(y_bits),
                                  perm["pair_pos"], topk_w, T, topk, n_shared)
    return dict(topk_ids=topk_ids, topk_w=topk_w, perm=perm, a1=a1, h=h, h_bits=h_bits,
                a2=a2, y=y, y_bits=y_bits, out=out, out_bits=out_bits)
