"""Grouped expert GEMMs (gate/up with SiLU(gate)*up, then down) and the combine.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[ATOM] "Stage D: MXFP4 Fused MoE": the MoE runs as two stages, stage 1 on the
fused gate/up weights (w13 with its E8M0 scale tensor), stage 2 on the down
weights (w2), the stage-2 outputs combined per token.  [GAUDI] "What was
built": per layer the experts' gate and up rows are concatenated into one
fused [384, ...] tensor.  [ATOM] "Choosing the Right Weight Layout": a gate
or up shard is 2048 output rows by 7168 K values, a down shard 7168 rows by
2048 K values.

Readings:
  * In the fused w13 tensor of an expert, rows 0..I-1 are gate, I..2I-1 up.
  * The activation between the stages is SiLU(gate) * up, SiLU(g) = g/(1+e^-g).
  * Rounding points: h (stage-1 output) and y (stage-2 output) are rounded to
    bf16; everything between them is float64 here.
  * The combine adds sum_j w[t,j] * y[pos(t,j)] over the routed slots in
    ascending j plus the shared-expert rows with weight 1, then rounds to bf16.
    Dropped pairs (pos = -1) contribute nothing.

Weight formats (dequantized per expert, float64):
  mx     codes [E, N, K/2] + E8M0 [E, N, K/32]         ([ATOM] "MXFP4 Tensor Anatomy")
  nvfp4  codes [E, N, K/2] + E4M3 [E, N, K/16] + fp32 tensor scale [E]
         ([NVFP4] "Weight Dequantization and Activation QDQ"; block 16 with
         E4M3 scales and one float32 tensor scale per expert and projection
         is the standard NVFP4 layout the page names)
  fp8    E4M3 codes [E, N, K] + float32 per-row channel scale [E, N]
         ([GAUDI] "Exact MXFP4 to FP8 per-channel conversion")
"""

import numpy as np

from . import formats as F


def dequant_expert(fmt, codes, scales, tensor_scale=None):
    """One expert's weight matrix [N, K] in float64."""
    if fmt == "mx":
        return F.mxfp4_dequant(codes, scales)
    if fmt == "nvfp4":
        return F.nvfp4_dequant(codes, scales, tensor_scale)
    if fmt == "fp8":
        return F.e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[:, None]
    raise ValueError(fmt)


def silu_mul(gu, I):
    g = gu[:, :I]
    u = gu[:, I:]
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def stage1_expert(a, w13, round_h=True):
    """a float64 [m, H], w13 float64 [2I, H] -> h [m, I] (bf16 values if round_h)."""
    I = w13.shape[0] // 2
    h = silu_mul(a @ w13.T, I)
    return F.bf16_round(h) if round_h else h


def stage2_expert(h, w2, round_y=True):
    """h float64 [m, I], w2 float64 [H, I] -> y [m, H] (bf16 values if round_y)."""
    y = h @ w2.T
    return F.bf16_round(y) if round_y else y


def grouped_stage(stage, a_sorted, expert_offsets, get_weight, rounding=True):
    """Run one stage over every expert segment of the sorted rows.

    a_sorted: float64 [n_rows, K] in sorted pair order.
    get_weight(e): float64 [N, K] weight matrix of expert e.
    Returns float64 [n_rows, N_out] (N_out = N/2 for stage 1).
    """
    offs = np.asarray(expert_offsets)
    Et = len(offs) - 1
    out = None
    for e in range(Et):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi == lo:
            continue
        w = get_weight(e)
        if stage == 1:
            r = stage1_expert(a_sorted[lo:hi], w, rounding)
        else:
            r = stage2_expert(a_sorted[lo:hi], w, rounding)
        if out is None:
            out = np.zeros((a_sorted.shape[0], r.shape[1]), dtype=np.float64)
        out[lo:hi] = r
    if out is None:
        out = np.zeros((a_sorted.shape[0], 0))
    return out


def moe_combine(y_sorted, pair_pos, topk_w, T, topk, n_shared):
    """-> (out float64 [T, H] before rounding, out bf16 bits [T, H])."""
    k = topk + n_shared
    H = y_sorted.shape[1]
    pos = np.asarray(pair_pos).reshape(T, k)
    w = np.asarray(topk_w, dtype=np.float64).reshape(T, topk)
    out = np.zeros((T, H), dtype=np.float64)
    for t in range(T):
        acc = np.zeros(H, dtype=np.float64)
        for j in range(k):
            p = pos[t, j]
            if p < 0:
                continue
            wt = w[t, j] if j < topk else 1.0
            acc = acc + wt * y_sorted[p]
        out[t] = acc
    return out, F.bf16_bits(out)
