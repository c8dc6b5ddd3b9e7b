"""End-to-end GPU parity of the whole layer (the seven calls chained) against the
oracle layer.  Routing ids and permutations bit-exact; the bf16 output within
the float tolerance of tests/parity.py.

At the full 7168/2048 width only the experts that the (oracle-computed)
routing selects get weights; every other expert's memory is left
uninitialized, so reading an expert that received no token would corrupt the
result.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import convert as OC
from oracle import layer as OL
from oracle import route as OR

from .parity import assert_bf16_close, assert_equal, assert_float_close
from .test_gpu_kernels import bf16_dev, bits_of, dev, host

pytestmark = pytest.mark.gpu


def build_weights(w, experts, wfmt, torch_empty_experts):
    """numpy weights for `experts` (dict e -> arrays) and device tensors with
    only those experts written."""
    Et = w.E + w.n_shared
    H, I = w.H, w.I
    np_w = {}
    dev_w = {}
    if wfmt in ("mx", "fp8"):
        dev_w["w13"] = torch.empty((Et, 2 * I, H // 2), dtype=torch.uint8, device="cuda")
        dev_w["w13_scale"] = torch.empty((Et, 2 * I, H // 32), dtype=torch.uint8, device="cuda")
        dev_w["w2"] = torch.empty((Et, H, I // 2), dtype=torch.uint8, device="cuda")
        dev_w["w2_scale"] = torch.empty((Et, H, I // 32), dtype=torch.uint8, device="cuda")
        if not torch_empty_experts:
            for t in dev_w.values():
                t.zero_()
        np_w = dict(w13={}, w13_scale={}, w2={}, w2_scale={})
        for e in experts:
            c13, s13 = synth.expert_mx(w, e, 13)
            c2, s2 = synth.expert_mx(w, e, 2)
            np_w["w13"][e], np_w["w13_scale"][e] = c13, s13
            np_w["w2"][e], np_w["w2_scale"][e] = c2, s2
            dev_w["w13"][e].copy_(torch.from_numpy(c13))
            dev_w["w13_scale"][e].copy_(torch.from_numpy(s13))
            dev_w["w2"][e].copy_(torch.from_numpy(c2))
            dev_w["w2_scale"][e].copy_(torch.from_numpy(s2))
    elif wfmt == "nvfp4":
        dev_w["w13"] = torch.empty((Et, 2 * I, H // 2), dtype=torch.uint8, device="cuda")
        dev_w["w13_scale"] = torch.empty((Et, 2 * I, H // 16), dtype=torch.uint8, device="cuda")
        dev_w["w2"] = torch.empty((Et, H, I // 2), dtype=torch.uint8, device="cuda")
        dev_w["w2_scale"] = torch.empty((Et, H, I // 16), dtype=torch.uint8, device="cuda")
        ts13 = np.zeros(Et, np.float32)
        ts2 = np.zeros(Et, np.float32)
        np_w = dict(w13={}, w13_scale={}, w2={}, w2_scale={}, w13_ts=ts13, w2_ts=ts2)
        for e in experts:
            c13, s13, t13 = synth.expert_nvfp4(w, e, 13)
            c2, s2, t2 = synth.expert_nvfp4(w, e, 2)
            np_w["w13"][e], np_w["w13_scale"][e], ts13[e] = c13, s13, t13
            np_w["w2"][e], np_w["w2_scale"][e], ts2[e] = c2, s2, t2
            dev_w["w13"][e].copy_(torch.from_numpy(c13))
            dev_w["w13_scale"][e].copy_(torch.from_numpy(s13))
            dev_w["w2"][e].copy_(torch.from_numpy(c2))
            dev_w["w2_scale"][e].copy_(torch.from_numpy(s2))
        dev_w["w13_ts"] = dev(ts13)
        dev_w["w2_ts"] = dev(ts2)
    if wfmt == "fp8":
        # FP8 experts are the oracle's exact conversion of the MXFP4 experts
        f13 = torch.empty((Et, 2 * I, H), dtype=torch.uint8, device="cuda")
        f2 = torch.empty((Et, H, I), dtype=torch.uint8, device="cuda")
        cs13 = torch.zeros((Et, 2 * I), dtype=torch.float32, device="cuda")
        cs2 = torch.zeros((Et, H), dtype=torch.float32, device="cuda")
        npf = dict(w13={}, w13_scale={}, w2={}, w2_scale={})
        for e in experts:
            r13 = OC.mxfp4_to_fp8_channel(np_w["w13"][e], np_w["w13_scale"][e])
            r2 = OC.mxfp4_to_fp8_channel(np_w["w2"][e], np_w["w2_scale"][e])
            assert r13["n_inexact"] == 0 and r2["n_inexact"] == 0
            npf["w13"][e], npf["w13_scale"][e] = r13["fp8"], r13["scale"]
            npf["w2"][e], npf["w2_scale"][e] = r2["fp8"], r2["scale"]
            f13[e].copy_(torch.from_numpy(r13["fp8"]))
            f2[e].copy_(torch.from_numpy(r2["fp8"]))
            cs13[e].copy_(torch.from_numpy(r13["scale"]))
            cs2[e].copy_(torch.from_numpy(r2["scale"]))
        np_w = npf
        dev_w = dict(w13=f13, w13_scale=cs13, w2=f2, w2_scale=cs2)
    return np_w, dev_w


# The inputs, weights and oracle results of the last (workload, T, seed,
# formats) case: the values do not depend on block_m or the weight layout
# (only the tile list does, which is not compared here), so the block_m
# variants of one case share them.
_CASE = {}


def _case(w, T, seed, afmt, wfmt):
    key = (id(w), T, seed, afmt, wfmt)
    if _CASE.get("key") != key:
        _CASE.clear()
        torch.cuda.empty_cache()
        logits = synth.router_logits(w, T, seed)
        bias = synth.router_bias(w)
        xb = synth.activations(w, T, seed)
        rid, rw = OR.moe_route(logits, bias, w.n_group, w.topk_group, w.topk)
        experts = sorted(set(rid.reshape(-1).tolist()) | set(range(w.E, w.E + w.n_shared)))
        np_w, dev_w = build_weights(w, experts, wfmt, torch_empty_experts=True)
        ref = OL.moe_layer(xb, logits, bias, np_w, E=w.E, n_shared=w.n_shared,
                           n_group=w.n_group, topk_group=w.topk_group, topk=w.topk, afmt=afmt,
                           wfmt=wfmt, block_m=16, topk_ids=rid, topk_w=rw)
        _CASE.update(key=key, logits=logits, bias=bias, xb=xb, rid=rid, rw=rw, dev_w=dev_w,
                     ref=ref)
    return _CASE


def run_layer(gpu_lib, w, T, afmt, wfmt, block_m, seed=0, fragment=True, fused=False):
    c = _case(w, T, seed, afmt, wfmt)
    logits, bias, xb, rid, rw, ref = c["logits"], c["bias"], c["xb"], c["rid"], c["rw"], c["ref"]
    cfg = gpu_lib.LayerConfig(H=w.H, I=w.I, E=w.E, n_shared=w.n_shared, n_group=w.n_group,
                              topk_group=w.topk_group, topk=w.topk, afmt=afmt, wfmt=wfmt,
                              block_m=block_m, fragment_layout=fragment, fused_decode=fused)
    layer = gpu_lib.MoELayer(cfg, c["dev_w"])
    b = layer.forward(bf16_dev(xb), dev(logits), dev(bias), keep=True)
    assert_equal(host(b["topk_ids"]), rid, "topk_ids")
    np.testing.assert_allclose(host(b["topk_w"]), rw, rtol=1e-6)
    assert_equal(host(b["perm"]["sorted_pairs"]), ref["perm"]["sorted_pairs"], "sorted_pairs")
    assert_equal(host(b["perm"]["pair_pos"]), ref["perm"]["pair_pos"], "pair_pos")
    n = int(ref["perm"]["expert_offsets"][-1])
    assert_bf16_close(bits_of(b["h"])[:n], ref["h"], "h")
    stats = assert_bf16_close(bits_of(b["out"]), ref["out"], "out")
    return stats


def test_layer_tiny_bf16_path(gpu_lib):
    run_layer(gpu_lib, synth.WORKLOADS["tiny"], 16, "bf16", "mx", 16)


def test_layer_tiny_bf16_path_rowmajor(gpu_lib):
    run_layer(gpu_lib, synth.WORKLOADS["tiny"], 16, "bf16", "mx", 16, fragment=False)


def test_layer_tiny_mx_path(gpu_lib):
    run_layer(gpu_lib, synth.WORKLOADS["tiny"], 16, "mx", "mx", 32)


@pytest.mark.parametrize("afmt,block_m", [("bf16", 16), ("mx", 32), ("mx", 192)])
def test_layer_empty_batch(gpu_lib, afmt, block_m):
    """T = 0: every call accepts the empty batch and the layer returns an empty
    output (the one-launch routing + permutation at decode sizes, the separate
    calls otherwise)."""
    w = synth.WORKLOADS["tiny"]
    # the 192-row tiles need output widths in whole 256 / 512-column blocks
    H, I = (512, 256) if block_m == 192 else (w.H, w.I)
    cfg = gpu_lib.LayerConfig(H=H, I=I, E=w.E, n_shared=w.n_shared, n_group=w.n_group,
                              topk_group=w.topk_group, topk=w.topk, afmt=afmt, wfmt="mx",
                              block_m=block_m)
    Et = w.E + w.n_shared
    g = np.random.default_rng(5)
    wts = {}
    for name, (N, K) in (("w13", (2 * I, H)), ("w2", (H, I))):
        wts[name] = dev(g.integers(0, 256, (Et, N, K // 2), dtype=np.uint8))
        wts[name + "_scale"] = dev(np.full((Et, N, K // 32), 127, np.uint8))
    layer = gpu_lib.MoELayer(cfg, wts)
    x = torch.zeros((0, H), dtype=torch.bfloat16, device="cuda")
    logits = torch.zeros((0, w.E), dtype=torch.float32, device="cuda")
    bias = torch.zeros(w.E, dtype=torch.float32, device="cuda")
    out = layer.forward(x, logits, bias)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, H)


@pytest.mark.parametrize("T,fused", [(1, True), (8, True), (16, True), (1, False), (8, False),
                                     (64, False)])
def test_layer_decode_full_width(gpu_lib, T, fused):
    """The decode layer at full width against the oracle: one launch
    (moe_decode_fused, up to 16 tokens) or the chain of calls."""
    run_layer(gpu_lib, synth.WORKLOADS["decode"], T, "bf16", "mx", 16, fused=fused)


def _fused_and_chain(gpu_lib, w, T, seed):
    """Outputs of the single-launch decode and of the chain of calls on the same
    inputs, and the fused layer's workspace after its calls."""
    c = _case(w, T, seed, "bf16", "mx")
    outs = []
    for fused in (True, False):
        cfg = gpu_lib.LayerConfig(H=w.H, I=w.I, E=w.E, n_shared=w.n_shared, n_group=w.n_group,
                                  topk_group=w.topk_group, topk=w.topk, afmt="bf16", wfmt="mx",
                                  block_m=16, fused_decode=fused)
        layer = gpu_lib.MoELayer(cfg, c["dev_w"])
        if fused:
            assert layer.fused_ok
            ws = layer.fused_ws
        b = layer.forward(bf16_dev(c["xb"]), dev(c["logits"]), dev(c["bias"]), keep=True)
        n = int(host(b["perm"]["expert_offsets"])[-1])
        nt = int(host(b["perm"]["n_tiles"])[0])
        outs.append({k: host(b[k]).copy() for k in ("topk_ids", "topk_w")} |
                    {k: host(b["perm"][k]).copy() for k in ("expert_offsets", "sorted_pairs",
                                                             "pair_pos", "n_tiles", "n_dropped")} |
                    {"tiles": host(b["perm"]["tiles"])[:nt].copy(),
                     "h": bits_of(b["h"])[:n].copy(), "y": bits_of(b["y"])[:n].copy(),
                     "out": bits_of(b["out"]).copy()})
    return outs[0], outs[1], host(ws).copy(), c


@pytest.mark.parametrize("wname,T", [("decode", 1), ("decode", 2), ("decode", 5), ("decode", 16),
                                     ("tiny", 1), ("tiny", 16)])
def test_decode_fused_matches_chain_bit_for_bit(gpu_lib, wname, T):
    """moe_decode_fused writes exactly what route+permute, both dq stages and
    the combine write (every output byte), the outputs match the oracle, and
    the workspace is back to its reusable state (counters at zero, no barrier
    timeout)."""
    w = synth.WORKLOADS[wname]
    f, u, ws, c = _fused_and_chain(gpu_lib, w, T, 0)
    for key in u:
        assert f[key].shape == u[key].shape and f[key].tobytes() == u[key].tobytes(), \
            f"{key}: fused and chained outputs differ"
    assert ws[0] == 0 and ws[2] == 0 and not ws[4:].any(), ws[:8]
    ref = c["ref"]
    assert_equal(f["topk_ids"], c["rid"], "topk_ids")
    assert_equal(f["pair_pos"], ref["perm"]["pair_pos"], "pair_pos")
    assert_bf16_close(f["out"], ref["out"], "out")


def test_decode_fused_repeated_calls(gpu_lib):
    """Many calls in a row on changing inputs: each equals the chain, and the
    barrier generation word advances once per call."""
    w = synth.WORKLOADS["decode"]
    cfg = gpu_lib.LayerConfig(H=w.H, I=w.I, E=w.E, n_shared=w.n_shared, n_group=w.n_group,
                              topk_group=w.topk_group, topk=w.topk, afmt="bf16", wfmt="mx",
                              block_m=16, fused_decode=True)
    ref_cfg = gpu_lib.LayerConfig(**{**cfg.__dict__, "fused_decode": False})
    T = 8
    c = _case(w, T, 0, "bf16", "mx")
    fused = gpu_lib.MoELayer(cfg, c["dev_w"])
    chain = gpu_lib.MoELayer(ref_cfg, c["dev_w"])
    g0 = int(host(fused.fused_ws)[1])
    bias = dev(c["bias"])
    rng = np.random.default_rng(7)
    for i in range(12):
        # same experts as the case (their weights are the only ones written):
        # permute the tokens and scale the logits of the routed experts up
        perm_t = rng.permutation(T)
        xb = c["xb"][perm_t]
        lg = c["logits"][perm_t].copy()
        x_d, l_d = bf16_dev(xb), dev(lg)
        a = bits_of(fused.forward(x_d, l_d, bias)).copy()
        b = bits_of(chain.forward(x_d, l_d, bias)).copy()
        assert a.tobytes() == b.tobytes(), f"call {i}"
    ws = host(fused.fused_ws)
    assert int(ws[1]) - g0 == 12 and ws[0] == 0 and ws[2] == 0 and not ws[4:].any()


def test_layer_decode_is_deterministic(gpu_lib):
    """The decode path (one-launch routing + permutation, split-K reduction in
    LDS in a fixed order): every output byte the same on a second run."""
    _twice(gpu_lib, synth.WORKLOADS["decode"], 8, "bf16", "mx", 16)


@pytest.mark.parametrize("block_m", [64, 192, 256])
def test_layer_prefill_path_full_width(gpu_lib, block_m):
    run_layer(gpu_lib, synth.WORKLOADS["prefill"], 24, "mx", "mx", block_m)




def sample_tokens(perm, k, T, E, n_shared, block_m, rng, n=32):
    """At least n tokens whose sorted rows cover: the first and last rows of the
    most loaded routed expert's first and last M tiles, both ends of a one-tile
    expert, both sides of the shared expert's first tile boundaries and of one
    in its middle; random tokens fill the rest."""
    offs = np.asarray(perm["expert_offsets"])
    sp = np.asarray(perm["sorted_pairs"])
    counts = np.diff(offs)
    big = int(np.argmax(counts[:E]))
    lo, hi = int(offs[big]), int(offs[big + 1])
    rows = [lo, lo + block_m - 1, lo + block_m, hi - block_m - 1, hi - block_m, hi - 1]
    one = np.flatnonzero((counts[:E] > 1) & (counts[:E] <= block_m))
    if one.size:
        rows += [int(offs[one[0]]), int(offs[one[0] + 1]) - 1]
    for sh in range(E, E + n_shared):
        o, c = int(offs[sh]), int(counts[sh])
        for edge in (block_m, 2 * block_m, (c // 2) // block_m * block_m):
            rows += [o + edge - 1, o + edge]
    rows = np.array([r for r in rows if 0 <= r < offs[-1]])
    toks = set((sp[rows] // k).tolist())
    while len(toks) < n:
        toks.add(int(rng.integers(T)))
    return np.array(sorted(toks))


# End-to-end drift bound of the MXFP4-activation layers.  h is re-quantized to
# MXFP4 between the stages, so a rounding-boundary flip of one h value (float32
# accumulation on the GPU against float64 in the oracle) moves a whole FP4
# code and compounds through stage 2; each stage is therefore held to the
# float tolerance on the GPU's own upstream outputs, and the end-to-end
# difference only to this looser bound.
END_TO_END_REL_L2 = 5e-3


def _full_size_layer(gpu_lib, wname, wfmt, seed, afmt="mx"):
    """The MXFP4-activation layer at a benchmarked size and launch configuration
    (192-row tiles, h quantized in the stage-1 epilogue; W8A8: 128-row tiles,
    h quantized per row by fp8_quant_per_token; the bf16 copy of h is also
    kept for the check).  Every token: routing ids and the permutation
    bit-exact.  At least 32 sampled tokens (sample_tokens), stage by stage on
    the GPU's own upstream outputs (a token's rows depend only on its own row,
    its routing and the weights):
      * the activation codes and scales bit-exact;
      * stage 1 (h, on whole 32-blocks of columns) against the oracle's stage 1;
      * the epilogue's MXFP4 codes of h (full rows) bit-exact against the
        oracle's quantizer applied to the GPU's h;
      * stage 2 (y, on 512 columns) against the oracle fed the GPU's full h
        codes;
      * the combine (full rows) against the oracle fed the GPU's y;
    and, on four of the tokens, the end-to-end output against the oracle layer
    within END_TO_END_REL_L2.  Only the checked weight rows are decoded, each
    expert once, so the oracle side stays within about a minute."""
    from oracle import formats as F
    from oracle import gemm as OG
    from oracle import permute as OP
    from oracle import quant as OQ
    w = synth.WORKLOADS[wname]
    T, Et, H, I = w.T, w.E + w.n_shared, w.H, w.I
    k = w.topk + w.n_shared
    logits = synth.router_logits(w, T, 0)
    bias = synth.router_bias(w)
    xb = synth.activations(w, T, 0)
    rid, rw = OR.moe_route(logits, bias, w.n_group, w.topk_group, w.topk)
    bm = 128 if afmt == "fp8" else 192
    perm = OP.moe_permute(rid, w.E, w.n_shared, bm)
    sub = sample_tokens(perm, k, T, w.E, w.n_shared, bm, np.random.default_rng(seed))
    need = set(rid[sub].reshape(-1).tolist()) | set(range(w.E, Et))
    np_w = dict(w13={}, w13_scale={}, w2={}, w2_scale={})
    if wfmt == "mx":
        dev_w = dict(w13=torch.empty((Et, 2 * I, H // 2), dtype=torch.uint8, device="cuda"),
                     w13_scale=torch.empty((Et, 2 * I, H // 32), dtype=torch.uint8, device="cuda"),
                     w2=torch.empty((Et, H, I // 2), dtype=torch.uint8, device="cuda"),
                     w2_scale=torch.empty((Et, H, I // 32), dtype=torch.uint8, device="cuda"))
        for e in range(Et):                  # every expert receives tokens at this size
            for proj, name in ((13, "w13"), (2, "w2")):
                c, sc = synth.expert_mx(w, e, proj)
                dev_w[name][e].copy_(torch.from_numpy(c))
                dev_w[name + "_scale"][e].copy_(torch.from_numpy(sc))
                if e in need:
                    np_w[name][e], np_w[name + "_scale"][e] = c, sc
    else:
        # E4M3 weights: uniform bytes without the NaN patterns, power-of-two
        # channel scales (any E4M3 operand exercises the same arithmetic as the
        # converted experts)
        dev_w = dict(w13=torch.empty((Et, 2 * I, H), dtype=torch.uint8, device="cuda"),
                     w13_scale=torch.empty((Et, 2 * I), dtype=torch.float32, device="cuda"),
                     w2=torch.empty((Et, H, I), dtype=torch.uint8, device="cuda"),
                     w2_scale=torch.empty((Et, H), dtype=torch.float32, device="cuda"))
        g = np.random.default_rng(97)
        for e in range(Et):
            for name, (N, K) in (("w13", (2 * I, H)), ("w2", (H, I))):
                c = g.integers(0, 256, (N, K), dtype=np.uint8)
                c[(c & 0x7F) == 0x7F] = 0x3C
                sc = np.ldexp(1.0, g.integers(-9, -3, N)).astype(np.float32)
                dev_w[name][e].copy_(torch.from_numpy(c))
                dev_w[name + "_scale"][e].copy_(torch.from_numpy(sc))
                if e in need:
                    np_w[name][e], np_w[name + "_scale"][e] = c, sc
    cfg = gpu_lib.LayerConfig(H=H, I=I, E=w.E, n_shared=w.n_shared, n_group=w.n_group,
                              topk_group=w.topk_group, topk=w.topk, afmt=afmt, wfmt=wfmt,
                              block_m=bm)
    layer = gpu_lib.MoELayer(cfg, dev_w)
    del dev_w
    b = layer.forward(bf16_dev(xb), dev(logits), dev(bias), keep=True)
    assert_equal(host(b["topk_ids"]), rid, "topk_ids")
    np.testing.assert_allclose(host(b["topk_w"]), rw, rtol=1e-6)
    assert_equal(host(b["perm"]["sorted_pairs"]), perm["sorted_pairs"], "sorted_pairs")
    assert_equal(host(b["perm"]["pair_pos"]), perm["pair_pos"], "pair_pos")
    assert_equal(host(b["perm"]["expert_offsets"]), perm["expert_offsets"], "expert_offsets")
    # the sampled tokens' sorted rows, slot by slot
    pos = np.asarray(perm["pair_pos"]).reshape(T, k)[sub]            # [n_sub, k]
    rows = pos.reshape(-1)
    row_e = np.searchsorted(perm["expert_offsets"], rows, side="right") - 1
    rows_d = torch.from_numpy(rows.astype(np.int64)).cuda()

    def chunked_rows(codes, scales):          # [K/128, P, 64|4] -> row-major [n, K/2], [n, K/32]
        c = codes.index_select(1, rows_d).permute(1, 0, 2).reshape(len(rows), -1)
        s_ = scales.index_select(1, rows_d).permute(1, 0, 2).reshape(len(rows), -1)
        return host(c), host(s_)

    def weight(name, e, wrows):
        """Rows wrows of expert e's dequantized weight (float64)."""
        return OG.dequant_expert(wfmt, np_w[name][e][wrows], np_w[name + "_scale"][e][wrows])

    def per_expert(name, wrows, inputs, fn):
        """fn(inputs of the rows of one expert, its weight rows) for every
        expert of the sampled rows, each expert's weights decoded once."""
        out = None
        for e in np.unique(row_e):
            idx = np.flatnonzero(row_e == e)
            r = fn(inputs[idx], weight(name, int(e), wrows))
            if out is None:
                out = np.empty((len(rows), r.shape[1]))
            out[idx] = r
        return out

    # checked columns: whole 32-blocks of h (first, last and random ones) and
    # 512 columns of y (first and last 64 and random ones); stage 2 still
    # consumes the GPU's full h rows
    g = np.random.default_rng(seed + 100)
    hb = np.unique(np.concatenate([[0, I // 32 - 1], g.choice(I // 32, 6, replace=False)]))
    h_cols = (hb[:, None] * 32 + np.arange(32)).reshape(-1)
    y_cols = np.unique(np.concatenate([np.arange(64), np.arange(H - 64, H),
                                       g.choice(H, 384, replace=False)]))
    if afmt == "fp8":
        # per-token FP8 codes of the sampled tokens (one row per token)
        sub_d = torch.from_numpy(sub.astype(np.int64)).cuda()
        xc = host(b["xq"].index_select(1, sub_d).permute(1, 0, 2).reshape(len(sub), -1))
        xs = host(b["xs"].index_select(0, sub_d))
        qc, qs = OQ.fp8_quant_per_token(xb[sub])
        assert_equal(xc, qc, "activation codes (sampled tokens)")
        assert_equal(xs, qs, "activation scales (sampled tokens)")
        a1 = np.repeat(F.e4m3_decode(qc) * qs.astype(np.float64)[:, None], k, axis=0)
    else:
        # activation codes of the sampled tokens (written to each of their rows)
        xc, xs = chunked_rows(b["xq"], b["xs"])
        qc, qs = OQ.mxfp4_quant_1x32(xb[sub])
        assert_equal(xc, np.repeat(qc, k, axis=0), "activation codes (sampled rows)")
        assert_equal(xs, np.repeat(qs, k, axis=0), "activation scales (sampled rows)")
        a1 = np.repeat(F.mxfp4_dequant(qc, qs), k, axis=0)
    print(f"[{wname}/{wfmt}] {len(sub)} tokens, {len(rows)} rows, "
          f"{len(np.unique(row_e))} experts: activation codes ok", flush=True)
    # stage 1 on the checked h columns (gate rows h_cols, up rows I + h_cols)
    h_gpu = host(b["h"].index_select(0, rows_d).view(torch.int16)).view(np.uint16)
    wr13 = np.concatenate([h_cols, I + h_cols])
    h_ref = per_expert("w13", wr13, a1, lambda a, wt: OG.stage1_expert(a, wt))
    assert_bf16_close(h_gpu[:, h_cols], h_ref, "h (sampled rows, checked columns)")
    print(f"[{wname}/{wfmt}] stage 1 ok", flush=True)
    if afmt == "fp8":
        # the per-row FP8 codes of h (fp8_quant_per_token on the GPU's h), full rows
        hc = host(b["hq"].index_select(1, rows_d).permute(1, 0, 2).reshape(len(rows), -1))
        hs = host(b["hs"].index_select(0, rows_d))
        rc, rs = OQ.fp8_quant_per_token(h_gpu)
        assert_equal(hc, rc, "h FP8 codes (sampled rows)")
        assert_equal(hs, rs, "h FP8 row scales (sampled rows)")
        a2 = F.e4m3_decode(hc) * hs.astype(np.float64)[:, None]
    else:
        # the epilogue's MXFP4 codes of h, full rows
        hc, hs = chunked_rows(b["hq"], b["hs"])
        rc, rs = OQ.mxfp4_quant_1x32(h_gpu)
        assert_equal(hc, rc, "h codes from the stage-1 epilogue (sampled rows)")
        assert_equal(hs, rs, "h scales from the stage-1 epilogue (sampled rows)")
        a2 = F.mxfp4_dequant(hc, hs)
    # stage 2 on the GPU's h codes, checked y columns
    y_gpu = host(b["y"].index_select(0, rows_d).view(torch.int16)).view(np.uint16)
    y_ref = per_expert("w2", y_cols, a2, lambda a, wt: OG.stage2_expert(a, wt))
    assert_bf16_close(y_gpu[:, y_cols], y_ref, "y (sampled rows, checked columns)")
    print(f"[{wname}/{wfmt}] h codes and stage 2 ok", flush=True)
    # the combine on the GPU's y, full rows (rows of token i are i*k .. i*k+k-1)
    out_ref, _ = OG.moe_combine(F.bf16_decode(y_gpu), np.arange(len(rows)), rw[sub], len(sub),
                                w.topk, w.n_shared)
    out_gpu = bits_of(b["out"])[sub]
    assert_bf16_close(out_gpu, out_ref, f"out ({len(sub)} sampled tokens, GPU y)")
    # end to end on four of the tokens
    e2e = sub[:: max(1, len(sub) // 4)][:4]
    ref = OL.moe_layer(xb[e2e], logits[e2e], bias, np_w, E=w.E, n_shared=w.n_shared,
                       n_group=w.n_group, topk_group=w.topk_group, topk=w.topk, afmt=afmt,
                       wfmt=wfmt, block_m=bm, topk_ids=rid[e2e], topk_w=rw[e2e])
    stats = assert_float_close(F.bf16_decode(bits_of(b["out"])[e2e]), F.bf16_round(ref["out"]),
                               "out end to end", rel_l2=END_TO_END_REL_L2, max_abs_rms=1.0)
    print(f"[{wname}/{wfmt}] combine ok; end-to-end rel-L2 {stats['rel_l2']:.2e}", flush=True)
    del layer, b
    torch.cuda.empty_cache()
    return np.diff(perm["expert_offsets"])


def test_layer_prefill_full_size_sampled(gpu_lib):
    """Prefill at T=8192 with uniform routing (see _full_size_layer)."""
    _full_size_layer(gpu_lib, "prefill", "mx", 11)


def test_layer_skewed_prefill_full_size_sampled(gpu_lib):
    """The skewed prefill at T=16384: Zipf(1.1) expert popularity, MXFP4 x MXFP4
    on 192-row tiles (see _full_size_layer).  The most loaded expert spans many
    M tiles; its first and last tiles are among the sampled rows."""
    counts = _full_size_layer(gpu_lib, "skewed", "mx", 12)
    assert counts[:384].max() > 8 * 192          # the routing really is skewed


def test_layer_w8a8_full_size_sampled(gpu_lib):
    """W8A8 at T=16384 with Zipf(1.1) routing: per-token FP8 activations x E4M3
    weights with power-of-two channel scales on the 128-row FP8 x FP8
    scaled-MFMA tiles (see _full_size_layer)."""
    _full_size_layer(gpu_lib, "skewed", "fp8", 14, afmt="fp8")


def test_layer_fp8_full_size_sampled(gpu_lib):
    """The FP8-weight layer at T=16384 with Zipf(1.1) routing: MXFP4 activations
    x E4M3 weights with power-of-two channel scales on the 192-row FP4 x FP8
    scaled-MFMA tiles (see _full_size_layer)."""
    _full_size_layer(gpu_lib, "skewed", "fp8", 13)


@pytest.mark.parametrize("bm", [128, 64])
def test_layer_nvfp4_full_size_sampled(gpu_lib, bm):
    """The NVFP4 emulation layer at the benchmarked size and launch configuration
    (T=2048, 128-row tiles; also 64-row tiles; activations in the f16 operand
    form), stage by stage
    on the GPU's own upstream outputs (the second QDQ's tensor scale spans all
    of h and couples every token, so each stage is checked on what the GPU fed
    it):
      * routing and permutation of every token bit-exact;
      * the activation QDQ of every token bit-exact;
      * stage 1 on sampled sorted rows against the oracle's stage 1;
      * the second QDQ of every row of the GPU's h bit-exact;
      * stage 2 on sampled sorted rows against the oracle run on the GPU's
        QDQ'd h;
      * the combine of sampled tokens against the oracle run on the GPU's y.
    Weights: uniform code bytes, positive finite E4M3 block scales, tensor
    scales U(0.01, 0.02)."""
    from oracle import formats as F
    from oracle import gemm as OG
    from oracle import permute as OP
    from oracle import quant as OQ
    w = synth.WORKLOADS["nvfp4"]
    T, Et, H, I = w.T, w.E + w.n_shared, w.H, w.I
    k = w.topk + w.n_shared
    logits = synth.router_logits(w, T, 0)
    bias = synth.router_bias(w)
    xb = synth.activations(w, T, 0)
    rid, rw = OR.moe_route(logits, bias, w.n_group, w.topk_group, w.topk)
    perm = OP.moe_permute(rid, w.E, w.n_shared, bm)
    offs = perm["expert_offsets"]
    counts = np.diff(offs)
    n_rows = int(offs[-1])
    # sampled sorted rows: the first and last rows of the most loaded expert
    # and of its first and last tiles, both ends of a one-tile expert, a
    # one-row expert if any, and random rows
    g = np.random.default_rng(98)
    big = int(np.argmax(counts))
    lo, hi = int(offs[big]), int(offs[big + 1])
    last0 = lo + (hi - lo - 1) // bm * bm          # first row of the last tile
    rows = [lo, lo + bm - 1, lo + bm, last0 - 1, last0, hi - 1]
    one = np.flatnonzero((counts > 1) & (counts <= bm))
    if one.size:
        rows += [int(offs[one[0]]), int(offs[one[0] + 1]) - 1]
    single = np.flatnonzero(counts == 1)
    if single.size:
        rows.append(int(offs[single[0]]))
    rows = np.unique(np.concatenate([rows, g.choice(n_rows, 16, replace=False)]))
    row_e = np.searchsorted(offs, rows, side="right") - 1
    toks = np.unique(perm["sorted_pairs"][rows] // k)
    dev_w = dict(w13=torch.empty((Et, 2 * I, H // 2), dtype=torch.uint8, device="cuda"),
                 w13_scale=torch.empty((Et, 2 * I, H // 16), dtype=torch.uint8, device="cuda"),
                 w2=torch.empty((Et, H, I // 2), dtype=torch.uint8, device="cuda"),
                 w2_scale=torch.empty((Et, H, I // 16), dtype=torch.uint8, device="cuda"))
    ts = {"w13": g.uniform(0.01, 0.02, Et).astype(np.float32),
          "w2": g.uniform(0.01, 0.02, Et).astype(np.float32)}
    kept = {"w13": {}, "w2": {}}
    sampled_experts = set(row_e.tolist())
    for e in range(Et):
        for name, (N, K) in (("w13", (2 * I, H)), ("w2", (H, I))):
            c = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
            sc = g.integers(0x01, 0x7F, (N, K // 16), dtype=np.uint8)   # positive finite E4M3
            dev_w[name][e].copy_(torch.from_numpy(c))
            dev_w[name + "_scale"][e].copy_(torch.from_numpy(sc))
            if e in sampled_experts:
                kept[name][e] = (c, sc)
    dev_w["w13_ts"], dev_w["w2_ts"] = dev(ts["w13"]), dev(ts["w2"])
    cfg = gpu_lib.LayerConfig(H=H, I=I, E=w.E, n_shared=w.n_shared, n_group=w.n_group,
                              topk_group=w.topk_group, topk=w.topk, afmt="nvfp4", wfmt="nvfp4",
                              block_m=bm)
    layer = gpu_lib.MoELayer(cfg, dev_w)
    assert layer.f16a, "the f16 operand path"
    del dev_w
    b = layer.forward(bf16_dev(xb), dev(logits), dev(bias), keep=True)
    assert_equal(host(b["topk_ids"]), rid, "topk_ids")
    np.testing.assert_allclose(host(b["topk_w"]), rw, rtol=1e-6)
    assert_equal(host(b["perm"]["sorted_pairs"]), perm["sorted_pairs"], "sorted_pairs")
    assert_equal(host(b["perm"]["pair_pos"]), perm["pair_pos"], "pair_pos")
    # activation QDQ of every token: the f16 operand times its power-of-two scale
    qx = OQ.nvfp4_qdq(xb)
    y_ref = F.bf16_decode(qx["y"])
    y_gpu = host(b["xq"]).astype(np.float64) * float(host(b["xs"])[0])
    assert np.array_equal(y_gpu, y_ref), "activation QDQ (f16 form)"
    del qx, y_gpu
    # stage 1 on sampled sorted rows
    tok = perm["sorted_pairs"][rows] // k
    h_all = bits_of(b["h"])[:n_rows]
    ref = np.empty((len(rows), I))
    for i, e in enumerate(row_e):
        c, sc = kept["w13"][int(e)]
        wd = OG.dequant_expert("nvfp4", c, sc, ts["w13"][e])
        ref[i] = OG.stage1_expert(y_ref[tok[i]][None, :], wd)[0]
    assert_bf16_close(h_all[rows], ref, "h (sampled rows)")
    del y_ref
    # the second QDQ over every row of the GPU's own h, bit-exact
    qh = OQ.nvfp4_qdq(h_all)
    a2_ref = F.bf16_decode(qh["y"])
    a2_gpu = host(b["hq"])[:n_rows].astype(np.float64) * float(host(b["hs"])[0])
    assert np.array_equal(a2_gpu, a2_ref), "second QDQ (f16 form) over every row of h"
    del qh, a2_gpu, h_all
    # stage 2 on sampled sorted rows, fed the QDQ'd GPU h
    y_all = bits_of(b["y"])
    ref = np.empty((len(rows), H))
    for i, e in enumerate(row_e):
        c, sc = kept["w2"][int(e)]
        wd = OG.dequant_expert("nvfp4", c, sc, ts["w2"][e])
        ref[i] = OG.stage2_expert(a2_ref[rows[i]][None, :], wd)[0]
    assert_bf16_close(y_all[rows], ref, "y (sampled rows)")
    del a2_ref
    # the combine of sampled tokens, fed the GPU's y
    pos = np.asarray(perm["pair_pos"]).reshape(T, k)[toks].reshape(-1)
    out_ref, _ = OG.moe_combine(F.bf16_decode(y_all), pos, rw[toks], len(toks), w.topk,
                                w.n_shared)
    assert_bf16_close(bits_of(b["out"])[toks], out_ref, f"out ({len(toks)} sampled tokens)")
    del layer, b, y_all
    torch.cuda.empty_cache()


def _twice(gpu_lib, w, T, afmt, wfmt, block_m):
    """Run the layer twice on the same inputs; every output byte must agree."""
    c = _case(w, T, 0, afmt, wfmt)
    cfg = gpu_lib.LayerConfig(H=w.H, I=w.I, E=w.E, n_shared=w.n_shared, n_group=w.n_group,
                              topk_group=w.topk_group, topk=w.topk, afmt=afmt, wfmt=wfmt,
                              block_m=block_m)
    layer = gpu_lib.MoELayer(cfg, c["dev_w"])
    runs = []
    for _ in range(2):
        b = layer.forward(bf16_dev(c["xb"]), dev(c["logits"]), dev(c["bias"]), keep=True)
        runs.append({k: host(b[k]).copy() for k in ("topk_ids", "topk_w")} |
                    {k: bits_of(b[k]).copy() for k in ("h", "y", "out")} |
                    {k: host(b["perm"][k]).copy() for k in ("sorted_pairs", "pair_pos", "tiles")})
    for k in runs[0]:
        assert runs[0][k].tobytes() == runs[1][k].tobytes(), f"{k} differs between two runs"


def test_layer_prefill_is_deterministic(gpu_lib):
    """Wide MXFP4 tiles with the epilogue quantization: no atomics anywhere."""
    _twice(gpu_lib, synth.WORKLOADS["prefill"], 24, "mx", "mx", 192)


@pytest.mark.parametrize("block_m", [16, 64, 128])
def test_layer_nvfp4_full_width(gpu_lib, block_m):
    run_layer(gpu_lib, synth.WORKLOADS["nvfp4"], 6, "nvfp4", "nvfp4", block_m)


@pytest.mark.parametrize("block_m", [64, 128])
def test_layer_nvfp4_is_deterministic(gpu_lib, block_m):
    """The NVFP4 tensor amax is an atomic maximum (order-free); the rest has no atomics."""
    _twice(gpu_lib, synth.WORKLOADS["nvfp4"], 6, "nvfp4", "nvfp4", block_m)


@pytest.mark.parametrize("block_m", [32, 64, 192])
def test_layer_fp8_full_width(gpu_lib, block_m):
    run_layer(gpu_lib, synth.WORKLOADS["skewed"], 6, "mx", "fp8", block_m)


def test_layer_w8a8_full_width(gpu_lib):
    """W8A8 (per-token FP8 activations, the oracle's exact FP8 conversion of the
    MXFP4 experts) at full width; several 128-row tiles per expert are covered
    by test_w8a8_gemm_parity and the full-size test."""
    run_layer(gpu_lib, synth.WORKLOADS["skewed"], 6, "fp8", "fp8", 128)


def test_layer_w8a8_is_deterministic(gpu_lib):
    _twice(gpu_lib, synth.WORKLOADS["skewed"], 6, "fp8", "fp8", 128)


def test_layer_fp8_is_deterministic(gpu_lib):
    """FP4 x FP8 192-row tiles: no atomics anywhere."""
    _twice(gpu_lib, synth.WORKLOADS["skewed"], 6, "mx", "fp8", 192)


@pytest.mark.parametrize("T", [8, 64])
def test_layer_expert_parallel_share(gpu_lib, T):
    """One of eight expert-parallel ranks: routed experts [0, 48) and the shared
    expert on this GPU, routing over all 384 experts, pairs routed elsewhere
    dropped by the permutation (and skipped by the combine)."""
    w = synth.WORKLOADS["decode"]
    E_loc = w.E // 8
    logits = synth.router_logits(w, T, 3)
    bias = synth.router_bias(w)
    xb = synth.activations(w, T, 3)
    H, I = w.H, w.I
    Et = E_loc + w.n_shared
    np_w = dict(w13={}, w13_scale={}, w2={}, w2_scale={})
    dev_w = dict(w13=torch.empty((Et, 2 * I, H // 2), dtype=torch.uint8, device="cuda"),
                 w13_scale=torch.empty((Et, 2 * I, H // 32), dtype=torch.uint8, device="cuda"),
                 w2=torch.empty((Et, H, I // 2), dtype=torch.uint8, device="cuda"),
                 w2_scale=torch.empty((Et, H, I // 32), dtype=torch.uint8, device="cuda"))
    for le, ge in enumerate(list(range(E_loc)) + list(range(w.E, w.E + w.n_shared))):
        c13, s13 = synth.expert_mx(w, ge, 13)
        c2, s2 = synth.expert_mx(w, ge, 2)
        np_w["w13"][le], np_w["w13_scale"][le], np_w["w2"][le], np_w["w2_scale"][le] = \
            c13, s13, c2, s2
        dev_w["w13"][le].copy_(torch.from_numpy(c13))
        dev_w["w13_scale"][le].copy_(torch.from_numpy(s13))
        dev_w["w2"][le].copy_(torch.from_numpy(c2))
        dev_w["w2_scale"][le].copy_(torch.from_numpy(s2))
    cfg = gpu_lib.LayerConfig(H=H, I=I, E=E_loc, n_shared=w.n_shared, n_group=w.n_group,
                              topk_group=w.topk_group, topk=w.topk, afmt="bf16", wfmt="mx",
                              block_m=16)
    layer = gpu_lib.MoELayer(cfg, dev_w)
    b = layer.forward(bf16_dev(xb), dev(logits), dev(bias), keep=True)
    ref = OL.moe_layer(xb, logits, bias, np_w, E=E_loc, n_shared=w.n_shared, n_group=w.n_group,
                       topk_group=w.topk_group, topk=w.topk, afmt="bf16", wfmt="mx", block_m=16)
    assert_equal(host(b["topk_ids"]), ref["topk_ids"].reshape(T, w.topk), "topk_ids")
    assert_equal(host(b["perm"]["pair_pos"]), ref["perm"]["pair_pos"], "pair_pos")
    assert int(host(b["perm"]["n_dropped"])[0]) == ref["perm"]["n_dropped"] > 0
    n = int(ref["perm"]["expert_offsets"][-1])
    assert_bf16_close(bits_of(b["h"])[:n], ref["h"], "h")
    assert_bf16_close(bits_of(b["out"]), ref["out"], "out")
