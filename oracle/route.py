"""Grouped sigmoid top-k routing with a correction bias.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[GAUDI] "What was built" (Quark MXFP4 repack): the model uses grouped top-k
routing with sigmoid scoring and a correction bias; [GAUDI] introduction: the
text tower is DeepSeek-V3 style with 384 routed experts.  The decode workload
groups the 384 experts in 8 groups and keeps 4 of them, top-8 experts.

The pages do not spell the rule out.  Reading (the DeepSeek-V3 scheme that
the pages name as the model family), with every decision taken in float32 so
that the ids are a function of float32 values only:
  1. s_e   = float32(1 / (1 + exp(-logit_e)))  evaluated in float64, rounded once.
  2. key_e = float32(s_e + bias_e)             (one IEEE float32 add).
     The bias steers the selection only; weights use s_e.
  3. With n_group > 1 the E experts form n_group groups of E/n_group
     contiguous ids.  A group's score is float32(top1 + top2) of its keys.
     The topk_group groups with the largest scores are kept; equal scores
     keep the lower group index.
  4. Among the kept experts the topk largest keys are selected in descending
     key order; equal keys select the lower expert id first.  This order is
     the slot order j = 0..topk-1.
  5. w_j = s_j / sum_i s_i (if renormalize) times routed_scale.
"""

import numpy as np


def sigmoid_fp32(logits):
    """float32 logits -> float32 scores, sigmoid evaluated in float64 and rounded once."""
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    return (1.0 / (1.0 + np.exp(-l))).astype(np.float32)


def _order_desc(values):
    """Indices sorting `values` descending, equal values by ascending index."""
    idx = np.arange(len(values))
    # lexsort sorts by the last key first: primary = -value, secondary = index
    return np.lexsort((idx, -values.astype(np.float64)))


def route_token(logit_row, bias, n_group, topk_group, topk, renormalize=True, routed_scale=1.0):
    """Route one token.  Returns (ids[topk] int32, weights[topk] float64)."""
    E = len(logit_row)
    s = sigmoid_fp32(logit_row)
    key = (s + np.asarray(bias, dtype=np.float32)).astype(np.float32)  # float32 add
    if n_group > 1:
        G = E // n_group
        gscore = np.empty(n_group, dtype=np.float32)
        for g in range(n_group):
            k = np.sort(key[g * G:(g + 1) * G].astype(np.float64))[::-1]
            gscore[g] = np.float32(np.float32(k[0]) + np.float32(k[1]))
        kept = _order_desc(gscore)[:topk_group]
        allowed = np.zeros(E, dtype=bool)
        for g in kept:
            allowed[g * G:(g + 1) * G] = True
    else:
        allowed = np.ones(E, dtype=bool)
    cand = np.nonzero(allowed)[0]
    order = cand[_order_desc(key[cand])]
    ids = order[:topk].astype(np.int32)
    sel = s[ids].astype(np.float64)
    if renormalize:
        w = sel / sel.sum()
    else:
        w = sel.copy()
    return ids, w * float(routed_scale)


def moe_route(logits, bias, n_group, topk_group, topk, renormalize=True, routed_scale=1.0):
    """logits float32 [T, E], bias float32 [E] -> ids int32 [T, topk], w float64 [T, topk]."""
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, topk), dtype=np.int32)
    w = np.empty((T, topk), dtype=np.float64)
    for t in range(T):
        ids[t], w[t] = route_token(logits[t], bias, n_group, topk_group, topk,
                                   renormalize, routed_scale)
    return ids, w
