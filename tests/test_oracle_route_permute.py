"""Pins of oracle/route.py and oracle/permute.py: brute force and invariants."""

import itertools

import numpy as np

from oracle import permute as P
from oracle import route as R


def _brute_route(logits, bias, n_group, topk_group, topk):
    """Exhaustive search: the group subset with the largest summed group score,
    then the expert subset inside it with the largest summed key."""
    E = len(logits)
    s = 1.0 / (1.0 + np.exp(-logits.astype(np.float64)))
    s32 = s.astype(np.float32)
    key = (s32 + bias.astype(np.float32)).astype(np.float32).astype(np.float64)
    G = E // n_group
    if n_group > 1:
        gs = []
        for g in range(n_group):
            kk = sorted(key[g * G:(g + 1) * G], reverse=True)
            gs.append(float(np.float32(np.float32(kk[0]) + np.float32(kk[1]))))
        best = max(itertools.combinations(range(n_group), topk_group),
                   key=lambda sub: sum(gs[g] for g in sub))
        allowed = [e for g in best for e in range(g * G, (g + 1) * G)]
    else:
        allowed = list(range(E))
    bsub = max(itertools.combinations(allowed, topk), key=lambda sub: sum(key[e] for e in sub))
    ids = sorted(bsub, key=lambda e: -key[e])
    sel = s32[ids].astype(np.float64)
    return np.array(ids), sel / sel.sum()


def test_route_brute_force_grouped():
    g = np.random.default_rng(10)
    for trial in range(60):
        E, n_group, tg, k = 16, 4, 2, 3
        logits = g.standard_normal(E).astype(np.float32)
        bias = (g.standard_normal(E) * 0.1).astype(np.float32)
        ids, w = R.route_token(logits, bias, n_group, tg, k)
        bids, bw = _brute_route(logits, bias, n_group, tg, k)
        assert list(ids) == list(bids), trial
        assert np.allclose(w, bw, rtol=0, atol=1e-15)


def test_route_brute_force_ungrouped():
    g = np.random.default_rng(11)
    for trial in range(40):
        logits = g.standard_normal(8).astype(np.float32)
        bias = (g.standard_normal(8) * 0.1).astype(np.float32)
        ids, w = R.route_token(logits, bias, 1, 1, 2)
        bids, bw = _brute_route(logits, bias, 1, 1, 2)
        assert list(ids) == list(bids)
        assert np.allclose(w, bw, atol=1e-15)


def test_route_group_score_is_top2_sum():
    # group 0 holds the single largest key but group 1 has the larger top-2 sum
    logits = np.array([4.0, -4, -4, -4, 2.0, 2.0, -4, -4], dtype=np.float32)
    ids, _ = R.route_token(logits, np.zeros(8, np.float32), n_group=2, topk_group=1, topk=2)
    assert sorted(ids) == [4, 5]
    ids, _ = R.route_token(logits, np.zeros(8, np.float32), n_group=1, topk_group=1, topk=2)
    assert list(ids) == [0, 4]


def test_route_ties_prefer_lower_index():
    logits = np.zeros(16, dtype=np.float32)
    ids, w = R.route_token(logits, np.zeros(16, np.float32), 4, 2, 5)
    assert list(ids) == [0, 1, 2, 3, 4]
    assert np.allclose(w, 0.2)
    logits = np.array([1, 2, 2, 1, 2, 0, 0, 0], dtype=np.float32)
    ids, _ = R.route_token(logits, np.zeros(8, np.float32), 1, 1, 3)
    assert list(ids) == [1, 2, 4]


def test_route_bias_selects_but_does_not_weight():
    logits = np.array([1.0, 0.5, 0.0, -0.5], dtype=np.float32)
    bias = np.array([0, 0, 5.0, 0], dtype=np.float32)
    ids, w = R.route_token(logits, bias, 1, 1, 2, renormalize=False)
    assert list(ids) == [2, 0]
    s = 1 / (1 + np.exp(-np.array([0.0, 1.0])))
    assert np.allclose(w, s.astype(np.float32).astype(np.float64), rtol=0, atol=0)


def test_route_weights_renormalized_and_scaled():
    g = np.random.default_rng(12)
    logits = g.standard_normal((20, 384)).astype(np.float32)
    bias = (g.standard_normal(384) * 0.1).astype(np.float32)
    ids, w = R.moe_route(logits, bias, 8, 4, 8, True, 2.5)
    assert np.allclose(w.sum(1), 2.5, atol=1e-12)
    for t in range(20):
        assert len(set(ids[t])) == 8
        groups = set(int(i) // 48 for i in ids[t])
        assert len(groups) <= 4


def test_sigmoid_fp32_exact_points():
    s = R.sigmoid_fp32(np.array([0.0, 200.0, -200.0], dtype=np.float32))
    assert s[0] == 0.5 and s[1] == 1.0 and s[2] == np.float32(1 / (1 + np.exp(200.0)))


# ---------------------------------------------------------------- permute

def _check_perm(ids, E, n_shared, bm):
    res = P.moe_permute(ids, E, n_shared, bm)
    T, topk = ids.shape
    k = topk + n_shared
    pe = P.pair_experts(ids, E, n_shared)
    nk = int(res["expert_offsets"][-1])
    sp = res["sorted_pairs"]
    pos = res["pair_pos"]
    # kept pairs are exactly those with a valid expert id
    valid = [p for p in range(T * k) if (p % k) >= topk or 0 <= pe[p] < E]
    assert nk == len(valid) and res["n_dropped"] == T * k - nk
    assert sorted(sp[:nk].tolist()) == valid and np.all(sp[nk:] == -1)
    # inverse relation
    for i in range(nk):
        assert pos[sp[i]] == i
    assert np.all(pos[[p for p in range(T * k) if p not in set(valid)]] == -1)
    # segments: experts non-decreasing, pairs ascending within an expert
    ex = pe[sp[:nk]]
    assert np.all(np.diff(ex) >= 0)
    for e in range(E + n_shared):
        lo, hi = res["expert_offsets"][e], res["expert_offsets"][e + 1]
        assert np.all(ex[lo:hi] == e)
        assert np.all(np.diff(sp[lo:hi]) > 0)
    # tiles
    tl = res["tiles"]
    exp_tiles = [(e, m) for e in range(E + n_shared)
                 for m in range(-(-int(res["counts"][e]) // bm))]
    assert [tuple(t) for t in tl] == exp_tiles
    assert res["n_tiles"] <= P.max_tiles(T, topk, E, n_shared, bm)
    return res


def test_permute_invariants_random():
    g = np.random.default_rng(13)
    for trial in range(30):
        T = int(g.integers(1, 40))
        E = int(g.integers(2, 20))
        topk = int(g.integers(1, min(E, 5) + 1))
        ids = np.stack([g.permutation(E)[:topk] for _ in range(T)]).astype(np.int32)
        _check_perm(ids, E, int(g.integers(0, 2)), int(g.choice([1, 4, 16])))


def test_permute_dropped_ids():
    ids = np.array([[0, -1], [5, 1], [1, 9]], dtype=np.int32)
    res = _check_perm(ids, 4, 1, 2)
    assert res["n_dropped"] == 3
    assert list(res["expert_offsets"]) == [0, 1, 3, 3, 3, 6]
    assert list(res["sorted_pairs"][:6]) == [0, 4, 6, 2, 5, 8]


def test_permute_hand_example():
    # T=3, topk=2, E=3, one shared expert (id 3), block_m=2
    ids = np.array([[2, 0], [0, 1], [2, 1]], dtype=np.int32)
    res = P.moe_permute(ids, 3, 1, 2)
    # pairs: p0 t0 e2, p1 t0 e0, p2 t0 e3, p3 t1 e0, p4 t1 e1, p5 t1 e3, p6 t2 e2, p7 t2 e1, p8 t2 e3
    assert list(res["expert_offsets"]) == [0, 2, 4, 6, 9]
    assert list(res["sorted_pairs"]) == [1, 3, 4, 7, 0, 6, 2, 5, 8]
    assert list(res["pair_pos"]) == [4, 0, 6, 1, 2, 7, 5, 3, 8]
    assert [tuple(t) for t in res["tiles"]] == [(0, 0), (1, 0), (2, 0), (3, 0), (3, 1)]


def test_max_tiles_bound_tight():
    # every token on its own expert with one row each: one tile per expert
    T, topk, E = 5, 1, 8
    ids = np.arange(T, dtype=np.int32)[:, None]
    res = P.moe_permute(ids, E, 0, 4)
    assert res["n_tiles"] == 5 == P.max_tiles(T, topk, E, 0, 4)
