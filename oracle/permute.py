"""Stable permutation of (token, slot) pairs by expert, and the tile list.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[NVFP4] "Memory Management": in the MoE path only the weights of dispatched
experts are touched.  [GAUDI] "Why MXFP4 decode was slow" and "What it taught
about Gaudi": cost must follow the routing (skip empty expert slots), not a
fixed slot count.  [K3] (A4W4 discussion): expert tiles carry padding.

Reading (the pages only say "sort/permute by expert"):
  * Every token has k = topk + n_shared slots.  Pair p = t*k + j.  Slots
    j < topk take the routed id; slot topk + i is shared expert E + i.
  * Pairs whose id lies outside [0, E) are dropped: they get pair_pos = -1
    and appear in no expert segment.
  * The kept pairs are sorted by expert id, stably (ascending p within an
    expert).  expert_offsets is the exclusive prefix sum of the counts over
    the E + n_shared experts, with the kept total as its last entry.
  * sorted_pairs[i] is the pair at sorted position i (-1 past the kept total);
    pair_pos[p] is the sorted position of pair p.
  * Tiles: for each expert with a non-zero count, ceil(count / block_m)
    entries (expert, m_tile) in expert order.  Empty experts get none.
"""

import numpy as np


def pair_experts(topk_ids, E, n_shared):
    """ids [T, topk] -> expert id of every pair, int64 [T*(topk+n_shared)]."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, topk = ids.shape
    k = topk + n_shared
    pe = np.empty((T, k), dtype=np.int64)
    pe[:, :topk] = ids
    for i in range(n_shared):
        pe[:, topk + i] = E + i
    return pe.reshape(-1)


def moe_permute(topk_ids, E, n_shared, block_m):
    T, topk = np.asarray(topk_ids).shape
    k = topk + n_shared
    P = T * k
    Et = E + n_shared
    pe = pair_experts(topk_ids, E, n_shared)
    valid = np.ones(P, dtype=bool)
    valid[:] = True
    for p in range(P):
        j = p % k
        if j < topk and not (0 <= pe[p] < E):
            valid[p] = False
    kept = [p for p in range(P) if valid[p]]
    order = sorted(kept, key=lambda p: (pe[p], p))
    counts = np.zeros(Et, dtype=np.int64)
    for p in kept:
        counts[pe[p]] += 1
    offsets = np.zeros(Et + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_pairs = np.full(P, -1, dtype=np.int32)
    sorted_pairs[:len(order)] = order
    pair_pos = np.full(P, -1, dtype=np.int32)
    for i, p in enumerate(order):
        pair_pos[p] = i
    tiles = []
    for e in range(Et):
        for mt in range(-(-int(counts[e]) // block_m)):
            tiles.append((e, mt))
    tiles = np.array(tiles, dtype=np.int32).reshape(-1, 2)
    return dict(expert_offsets=offsets, sorted_pairs=sorted_pairs, pair_pos=pair_pos,
                tiles=tiles, n_tiles=len(tiles), n_dropped=int(P - len(kept)),
                counts=counts)


def max_tiles(T, topk, E, n_shared, block_m):
    """Upper bound on the tile count for any routing of T tokens.

    sum_e ceil(c_e / bm) <= (sum_e c_e + n_nonempty * (bm - 1)) / bm, with
    sum_e c_e <= T*k and n_nonempty <= min(E + n_shared, T*k).
    """
    P = T * (topk + n_shared)
    ne = min(E + n_shared, P)
    return (P + ne * (block_m - 1)) // block_m
