"""Pins of oracle/gemm.py and oracle/layer.py.

* brute-force Python loops on tiny shapes (no matmul);
* one expert with weight 1 is the textbook SwiGLU MLP (two matmuls);
* dense equivalence: routing every token to every expert (topk = E, one group,
  renormalized) equals sum_e w_e * MLP_e(x) computed densely with no routing,
  permutation or combine machinery.
"""

import math

import numpy as np

import synth
from oracle import formats as F
from oracle import gemm as G
from oracle import layer as L
from oracle import route as R


def _tiny_weights(E, H, I, seed, lo=-6, hi=0):
    g = np.random.default_rng(seed)
    w = dict(w13=g.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8),
             w13_scale=(127 + g.integers(lo, hi + 1, (E, 2 * I, H // 32))).astype(np.uint8),
             w2=g.integers(0, 256, (E, H, I // 2), dtype=np.uint8),
             w2_scale=(127 + g.integers(lo, hi + 1, (E, H, I // 32))).astype(np.uint8))
    return w


def test_stage_brute_force_loops():
    g = np.random.default_rng(30)
    m, H, I = 3, 64, 32
    a = F.bf16_decode(synth.bf16_from_f32(g.standard_normal((m, H)).astype(np.float32)))
    w = _tiny_weights(1, H, I, 31)
    w13 = G.dequant_expert("mx", w["w13"][0], w["w13_scale"][0])
    w2 = G.dequant_expert("mx", w["w2"][0], w["w2_scale"][0])
    # dequant by hand: table[code & 7] * sign * 2^(scale - 127), low nibble first
    table = [0, .5, 1, 1.5, 2, 3, 4, 6]
    for n in range(0, 2 * I, 7):
        for kk in range(0, H, 5):
            byte = int(w["w13"][0, n, kk // 2])
            c = (byte >> 4) if kk % 2 else (byte & 15)
            v = table[c & 7] * (-1 if c & 8 else 1) * 2.0 ** (int(w["w13_scale"][0, n, kk // 32]) - 127)
            assert w13[n, kk] == v
    h = G.stage1_expert(a, w13, round_h=False)
    y = G.stage2_expert(h, w2, round_y=False)
    for r in range(m):
        for n in range(I):
            gs = sum(a[r, kk] * w13[n, kk] for kk in range(H))
            us = sum(a[r, kk] * w13[I + n, kk] for kk in range(H))
            want = gs / (1 + math.exp(-gs)) * us
            assert abs(h[r, n] - want) <= 1e-12 * max(1, abs(want))
        for n in range(H):
            want = sum(h[r, kk] * w2[n, kk] for kk in range(I))
            assert abs(y[r, n] - want) <= 1e-12 * max(1, abs(want))


def test_single_expert_is_textbook_swiglu():
    g = np.random.default_rng(32)
    T, H, I = 5, 64, 32
    xb = synth.bf16_from_f32(g.standard_normal((T, H)).astype(np.float32))
    w = _tiny_weights(1, H, I, 33)
    r = L.moe_layer(xb, None, None, w, E=1, n_shared=0, n_group=1, topk_group=1, topk=1,
                    afmt="bf16", wfmt="mx", rounding=False,
                    topk_ids=np.zeros((T, 1), np.int32), topk_w=np.ones((T, 1)))
    x = F.bf16_decode(xb)
    W13 = F.mxfp4_dequant(w["w13"][0], w["w13_scale"][0])
    W2 = F.mxfp4_dequant(w["w2"][0], w["w2_scale"][0])
    gate = np.matmul(x, W13[:I].T)
    up = np.matmul(x, W13[I:].T)
    ref = np.matmul(gate * (1 / (1 + np.exp(-gate))) * up, W2.T)
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-9)


def test_dense_equivalence_invariant():
    g = np.random.default_rng(34)
    T, H, I, E = 6, 64, 32, 5
    xb = synth.bf16_from_f32(g.standard_normal((T, H)).astype(np.float32))
    logits = g.standard_normal((T, E)).astype(np.float32)
    bias = (g.standard_normal(E) * 0.1).astype(np.float32)
    w = _tiny_weights(E, H, I, 35)
    for rounding in (False, True):
        r = L.moe_layer(xb, logits, bias, w, E=E, n_shared=0, n_group=1, topk_group=1, topk=E,
                        afmt="bf16", wfmt="mx", rounding=rounding)
        # dense: every expert on every token, weights = renormalized sigmoid scores
        x = F.bf16_decode(xb)
        s = R.sigmoid_fp32(logits).astype(np.float64)
        wd = s / s.sum(1, keepdims=True)
        dense = np.zeros((T, H))
        for e in range(E):
            W13 = F.mxfp4_dequant(w["w13"][e], w["w13_scale"][e])
            W2 = F.mxfp4_dequant(w["w2"][e], w["w2_scale"][e])
            gu = x @ W13.T
            h = gu[:, :I] / (1 + np.exp(-gu[:, :I])) * gu[:, I:]
            if rounding:
                h = F.bf16_round(h)
            y = h @ W2.T
            if rounding:
                y = F.bf16_round(y)
            dense += wd[:, e:e + 1] * y
        assert np.allclose(r["out"], dense, rtol=1e-12, atol=1e-12 * np.abs(dense).max())


def test_combine_brute_force_with_shared_and_dropped():
    g = np.random.default_rng(36)
    T, topk, H = 4, 2, 8
    k = topk + 1
    y = g.standard_normal((T * k, H))
    pos = g.permutation(T * k).astype(np.int32)
    pos[5] = -1
    w = g.uniform(0, 1, (T, topk))
    out, bits = G.moe_combine(y, pos, w, T, topk, 1)
    for t in range(T):
        want = np.zeros(H)
        for j in range(k):
            p = pos[t * k + j]
            if p >= 0:
                want += (w[t, j] if j < topk else 1.0) * y[p]
        assert np.allclose(out[t], want, rtol=0, atol=1e-15)
    assert np.array_equal(bits, F.bf16_bits(out))


def test_nvfp4_and_fp8_dequant_paths():
    g = np.random.default_rng(37)
    codes = g.integers(0, 256, (4, 16), dtype=np.uint8)
    sc = synth.e4m3_from_f32(np.abs(g.standard_normal((4, 2))).astype(np.float32))
    w = G.dequant_expert("nvfp4", codes, sc, np.float32(0.0125))
    c = F.unpack_fp4(codes)
    for n in range(4):
        for kk in range(32):
            want = F.e2m1_decode(c[n, kk]) * F.e4m3_decode(sc[n, kk // 16]) * np.float64(np.float32(0.0125))
            assert w[n, kk] == want
    f8 = g.integers(0, 0x7E, (3, 8), dtype=np.uint8)
    cs = np.array([0.5, 2.0 ** -20, 8.0], dtype=np.float32)
    w = G.dequant_expert("fp8", f8, cs)
    assert np.array_equal(w, F.e4m3_decode(f8) * cs[:, None].astype(np.float64))


# --------------------------------------------------------------------------
# The activation chaining of the layer (afmt "mx" and "nvfp4"), pinned by a
# per-token, per-slot brute force that uses no permutation, no grouped stage
# and no sorted-row order.  [ATOM] "Stage B: Dynamic Activation Quantization":
# the live activations of each GEMM are quantized at run time, so h is
# re-quantized before stage 2.  [NVFP4] "Weight Dequantization and Activation
# QDQ": a QDQ round trip before each GEMM; the dynamic tensor scale of stage 2
# covers every (token, slot) row of h at once.
# --------------------------------------------------------------------------

def _chain_weights(wfmt, Et, H, I, seed):
    g = np.random.default_rng(seed)
    if wfmt == "mx":
        return _tiny_weights(Et, H, I, seed)
    if wfmt == "fp8":
        w = {}
        for name, (N, K) in (("w13", (2 * I, H)), ("w2", (H, I))):
            c = g.integers(0, 256, (Et, N, K), dtype=np.uint8)
            c[(c & 0x7F) == 0x7F] = 0x38
            w[name] = c
            w[name + "_scale"] = np.ldexp(1.0, g.integers(-6, -2, (Et, N))).astype(np.float32)
        return w
    w = {}
    for name, (N, K) in (("w13", (2 * I, H)), ("w2", (H, I))):
        w[name] = g.integers(0, 256, (Et, N, K // 2), dtype=np.uint8)
        w[name + "_scale"] = synth.e4m3_from_f32(
            np.abs(g.standard_normal((Et, N, K // 16))).astype(np.float32))
        w[name + "_ts"] = g.uniform(0.01, 0.02, Et).astype(np.float32)
    return w


def _chain_brute_force(xb, ids, wts, w, afmt, wfmt, E, n_shared, I, requant_h=True):
    """out float64 [T, H] of the layer, one token and one slot at a time."""
    from oracle import quant as Q
    T = xb.shape[0]
    topk = ids.shape[1]

    def weight(name, e):
        if wfmt == "mx":
            return F.mxfp4_dequant(w[name][e], w[name + "_scale"][e])
        if wfmt == "fp8":
            return F.e4m3_decode(w[name][e]) * w[name + "_scale"][e].astype(np.float64)[:, None]
        return F.nvfp4_dequant(w[name][e], w[name + "_scale"][e], w[name + "_ts"][e])

    def qdq_rows(rows_bits, s_t=None):
        if afmt == "mx":
            return [Q.mxfp4_qdq_values(r[None])[0] for r in rows_bits]
        if afmt == "fp8":
            return [Q.fp8_qdq_values(r[None])[0] for r in rows_bits]
        return [F.bf16_decode(Q.nvfp4_qdq(r[None], tensor_scale_in=s_t)["y"])[0]
                for r in rows_bits]

    # stage-1 input: each token alone, the NVFP4 tensor scale over all of x
    s1 = Q.nvfp4_qdq(xb)["tensor_scale"] if afmt == "nvfp4" else None
    a = qdq_rows(list(xb), s1)
    slots = [(t, j, int(ids[t, j]) if j < topk else E + (j - topk))
             for t in range(T) for j in range(topk + n_shared)]
    h_bits = []
    for t, j, e in slots:
        w13 = weight("w13", e)
        gate = np.array([sum(w13[n, q] * a[t][q] for q in range(w13.shape[1]))
                         for n in range(I)])
        up = np.array([sum(w13[I + n, q] * a[t][q] for q in range(w13.shape[1]))
                       for n in range(I)])
        h_bits.append(F.bf16_bits(gate / (1.0 + np.exp(-gate)) * up))
    if not requant_h:
        a2 = [F.bf16_decode(hb) for hb in h_bits]
    else:
        # the NVFP4 stage-2 tensor scale spans every row of h
        s2 = Q.nvfp4_qdq(np.stack(h_bits))["tensor_scale"] if afmt == "nvfp4" else None
        a2 = qdq_rows(h_bits, s2)
    out = np.zeros((T, xb.shape[1]))
    for (t, j, e), hv in zip(slots, a2):
        y = F.bf16_round(weight("w2", e) @ hv)
        out[t] += (wts[t, j] if j < topk else 1.0) * y
    return out


def _check_chain(afmt, wfmt, seed):
    g = np.random.default_rng(seed)
    T, H, I, E, n_shared, topk = 5, 64, 32, 6, 1, 2
    xb = synth.bf16_from_f32(g.standard_normal((T, H)).astype(np.float32))
    logits = g.standard_normal((T, E)).astype(np.float32)
    bias = (g.standard_normal(E) * 0.1).astype(np.float32)
    w = _chain_weights(wfmt, E + n_shared, H, I, seed + 1)
    r = L.moe_layer(xb, logits, bias, w, E=E, n_shared=n_shared, n_group=1, topk_group=1,
                    topk=topk, afmt=afmt, wfmt=wfmt)
    want = _chain_brute_force(xb, r["topk_ids"], r["topk_w"], w, afmt, wfmt, E, n_shared, I)
    scale = np.abs(want).max()
    assert np.allclose(r["out"], want, rtol=1e-12, atol=1e-12 * scale)
    # the re-quantization of h is visible at this size: without it the layer differs
    plain = _chain_brute_force(xb, r["topk_ids"], r["topk_w"], w, afmt, wfmt, E, n_shared, I,
                               requant_h=False)
    assert np.abs(plain - want).max() > 1e-3 * scale


def test_layer_mx_activation_chain_brute_force():
    _check_chain("mx", "mx", 40)


def test_layer_nvfp4_activation_chain_brute_force():
    _check_chain("nvfp4", "nvfp4", 42)


def test_layer_fp8_activation_chain_brute_force():
    """W8A8: per-token FP8 activations before stage 1, per-row FP8 of h before
    stage 2, FP8 weights with per-channel scales."""
    _check_chain("fp8", "fp8", 44)
