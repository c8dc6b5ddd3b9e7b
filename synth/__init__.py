"""Seeded synthetic inputs for the block-scaled FP4 MoE layer.

This module serves both the CPU oracle's tests and the HIP library's tests
and benchmark.  It holds none of the layer's arithmetic: only random draws
(NumPy PCG64 streams keyed by SeedSequence([workload_id, tensor_id, ...])) and
dtype casts done by library routines (float32 -> bf16 and float32 -> E4M3 by
torch's round-to-nearest-even casts).

Workloads (shapes of the DeepSeek-V3 / Kimi K2 MoE layer that the pages
describe: 384 routed experts, top-8, hidden 7168, expert intermediate 2048):
  1 tiny    T=16, H=256, I=128, 8 experts top-2, no shared expert
  2 decode  T in {1, 8, 64}, 384 experts + 1 shared, groups 8 keep 4, top-8
  3 prefill T=8192, uniform routing, MXFP4 activations
  4 nvfp4   T=2048, 384 experts top-8, NVFP4 weights, QDQ activations
  5 skewed  T=16384, Zipf(1.1) expert popularity; MXFP4 -> FP8 conversion
"""

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    T: int
    H: int
    I: int
    E: int
    n_shared: int
    n_group: int
    topk_group: int
    topk: int
    scale_lo: int            # E8M0 code range 127+lo .. 127+hi (inclusive)
    scale_hi: int
    bias_std: float
    afmt: str                # activation path: bf16 | mx | nvfp4
    wfmt: str                # weight format: mx | nvfp4 | fp8
    routing: str = "normal"  # normal | zipf
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny": Workload(1, "tiny", 16, 256, 128, 8, 0, 1, 1, 2, -6, 0, 0.1, "bf16", "mx"),
    "decode": Workload(2, "decode", 8, 7168, 2048, 384, 1, 8, 4, 8, -8, -2, 0.1, "bf16", "mx"),
    "prefill": Workload(3, "prefill", 8192, 7168, 2048, 384, 1, 8, 4, 8, -8, -2, 0.0, "mx", "mx"),
    "nvfp4": Workload(4, "nvfp4", 2048, 7168, 2048, 384, 0, 8, 4, 8, 0, 0, 0.1, "nvfp4", "nvfp4"),
    "skewed": Workload(5, "skewed", 16384, 7168, 2048, 384, 1, 8, 4, 8, -8, -2, 0.0, "mx", "mx",
                       routing="zipf"),
}

# tensor ids of the seed streams
TID_LOGITS, TID_BIAS, TID_X = 1, 2, 3
TID_W13, TID_W13S, TID_W2, TID_W2S, TID_W13TS, TID_W2TS = 10, 11, 12, 13, 14, 15
TID_ZIPF_PERM = 20


def rng(*key):
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def bf16_from_f32(a):
    """float32 array -> bf16 bit patterns (uint16), by torch's RNE cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def e4m3_from_f32(a):
    """float32 array -> OCP E4M3FN bytes, by torch's RNE cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def normal_bf16(shape, *key, std=1.0):
    return bf16_from_f32(rng(*key).standard_normal(shape, dtype=np.float32) * np.float32(std))


def random_bytes(shape, *key):
    return rng(*key).integers(0, 256, size=shape, dtype=np.uint8)


def e8m0_scales(shape, lo, hi, *key):
    return (127 + rng(*key).integers(lo, hi + 1, size=shape)).astype(np.uint8)


def router_logits(w: Workload, T, seed=0):
    """float32 [T, E] router logits (the router GEMM is outside the FP4 path)."""
    if w.routing == "zipf":
        # Gumbel-top-k over log-popularity: Zipf(s=1.1) over randomly permuted ranks.
        perm = rng(w.wid, TID_ZIPF_PERM).permutation(w.E)
        ranks = np.empty(w.E, dtype=np.float64)
        ranks[perm] = np.arange(1, w.E + 1)
        logp = -1.1 * np.log(ranks)
        g = rng(w.wid, TID_LOGITS, seed).gumbel(size=(T, w.E))
        return (logp[None, :] + g).astype(np.float32)
    return rng(w.wid, TID_LOGITS, seed).standard_normal((T, w.E), dtype=np.float32)


def router_bias(w: Workload):
    if w.bias_std == 0.0:
        return np.zeros(w.E, dtype=np.float32)
    return (rng(w.wid, TID_BIAS).standard_normal(w.E, dtype=np.float32)
            * np.float32(w.bias_std)).astype(np.float32)


def activations(w: Workload, T, seed=0):
    return normal_bf16((T, w.H), w.wid, TID_X, seed)


def expert_mx(w: Workload, e, proj, layer=0):
    """One expert's MXFP4 weight: (codes [N, K/2], E8M0 scales [N, K/32]).

    proj 13: fused gate/up [2I, H];  proj 2: down [H, I]."""
    N, K = (2 * w.I, w.H) if proj == 13 else (w.H, w.I)
    tc, ts = (TID_W13, TID_W13S) if proj == 13 else (TID_W2, TID_W2S)
    codes = random_bytes((N, K // 2), w.wid, tc, layer, e)
    scales = e8m0_scales((N, K // 32), w.scale_lo, w.scale_hi, w.wid, ts, layer, e)
    return codes, scales


def expert_nvfp4(w: Workload, e, proj, layer=0):
    """One expert's NVFP4 weight: (codes [N, K/2], E4M3 scales [N, K/16], tensor scale)."""
    N, K = (2 * w.I, w.H) if proj == 13 else (w.H, w.I)
    tc, ts, tt = ((TID_W13, TID_W13S, TID_W13TS) if proj == 13 else (TID_W2, TID_W2S, TID_W2TS))
    codes = random_bytes((N, K // 2), w.wid, tc, layer, e)
    sc = e4m3_from_f32(np.abs(rng(w.wid, ts, layer, e).standard_normal((N, K // 16),
                                                                     dtype=np.float32)))
    tsc = np.float32(rng(w.wid, tt, layer, e).uniform(0.01, 0.02))
    return codes, sc, tsc


def spanned_scales(n_rows, n_blocks, *key, top_lo=-4, top_hi=0, span_lo=1, span_hi=9):
    """E8M0 rows whose codes span exactly U{span_lo..span_hi} binades.

    Top code 127+U{top_lo..top_hi}; one block at the top, one at the bottom
    of the span, the rest uniform in between."""
    g = rng(*key)
    top = 127 + g.integers(top_lo, top_hi + 1, size=n_rows)
    span = g.integers(span_lo, span_hi + 1, size=n_rows)
    u = g.integers(0, 1 << 30, size=(n_rows, n_blocks))
    s = top[:, None] - (u % (span[:, None] + 1))
    pos = g.permuted(np.tile(np.arange(n_blocks), (n_rows, 1)), axis=1)[:, :2]
    rows = np.arange(n_rows)
    s[rows, pos[:, 0]] = top
    s[rows, pos[:, 1]] = top - span
    return s.astype(np.uint8), span
