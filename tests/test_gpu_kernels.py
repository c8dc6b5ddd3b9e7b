"""GPU parity of every C-ABI entry point against the CPU oracle.

Integer / code outputs must match bit for bit; float outputs follow the
tolerances in tests/parity.py.  Inputs come from seeded generators (synth)
or are built by hand for edge cases; expected values come from oracle/ only.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import convert as OC
from oracle import formats as F
from oracle import gemm as OG
from oracle import permute as OP
from oracle import quant as OQ
from oracle import route as OR

from .parity import assert_bf16_close, assert_equal, assert_float_close
from .test_oracle_convert import load_convert_golden

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bf16_dev(bits):
    return dev(np.asarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def bits_of(t):
    return host(t.view(torch.int16)).view(np.uint16)


# ------------------------------------------------------------------ routing

ROUTE_CASES = [
    # (T, E, n_group, topk_group, topk, bias_std, seed)
    (16, 8, 1, 1, 2, 0.1, 1),
    (64, 384, 8, 4, 8, 0.1, 2),
    (777, 384, 8, 4, 8, 0.1, 3),
    (33, 256, 8, 4, 8, 0.0, 4),
    (5, 1024, 16, 2, 32, 0.5, 5),
    # group layouts: lanes per group 16 and 32, one expert per lane, an
    # experts-per-lane bound above ceil(E/64), groups that are not lane runs
    (40, 384, 4, 2, 8, 0.1, 6), (40, 384, 2, 1, 8, 0.1, 7), (20, 64, 2, 1, 4, 0.2, 8),
    (20, 128, 4, 2, 6, 0.1, 9), (12, 512, 8, 3, 10, 0.1, 10), (9, 320, 8, 4, 8, 0.1, 11),
    (7, 600, 6, 3, 8, 0.1, 12),
]


@pytest.mark.parametrize("case", ROUTE_CASES)
def test_route_parity(gpu_lib, case):
    T, E, ng, tg, k, bstd, seed = case
    g = np.random.default_rng(seed)
    logits = g.standard_normal((T, E), dtype=np.float32)
    bias = (g.standard_normal(E, dtype=np.float32) * np.float32(bstd)).astype(np.float32)
    ids, w = gpu_lib.moe_route(dev(logits), dev(bias), ng, tg, k)
    rid, rw = OR.moe_route(logits, bias, ng, tg, k)
    assert_equal(host(ids), rid, "topk_ids")
    np.testing.assert_allclose(host(w), rw, rtol=1e-6, atol=0)


def test_route_ties_and_options(gpu_lib):
    T, E = 3, 384
    logits = np.zeros((T, E), dtype=np.float32)
    logits[1, 100:110] = 1.0             # ties inside one group
    logits[2, ::7] = -1.0
    bias = np.zeros(E, dtype=np.float32)
    for renorm, scale in ((True, 1.0), (False, 2.5)):
        ids, w = gpu_lib.moe_route(dev(logits), dev(bias), 8, 4, 8, renorm, scale)
        rid, rw = OR.moe_route(logits, bias, 8, 4, 8, renorm, scale)
        assert_equal(host(ids), rid, "topk_ids ties")
        np.testing.assert_allclose(host(w), rw, rtol=1e-6)
    assert list(rid[0]) == list(range(8))


def test_route_decode_workload(gpu_lib):
    w = synth.WORKLOADS["decode"]
    for T in (1, 8, 64):
        logits = synth.router_logits(w, T)
        bias = synth.router_bias(w)
        ids, wt = gpu_lib.moe_route(dev(logits), dev(bias), w.n_group, w.topk_group, w.topk)
        rid, rw = OR.moe_route(logits, bias, w.n_group, w.topk_group, w.topk)
        assert_equal(host(ids), rid, f"decode T={T}")
        np.testing.assert_allclose(host(wt), rw, rtol=1e-6)


# ------------------------------------------------------------------ permute

def _perm_check(gpu_lib, ids, E, n_shared, bm):
    out = gpu_lib.moe_permute(dev(ids), E, n_shared, bm)
    ref = OP.moe_permute(ids, E, n_shared, bm)
    assert_equal(host(out["expert_offsets"]), ref["expert_offsets"], "expert_offsets")
    assert_equal(host(out["sorted_pairs"]), ref["sorted_pairs"], "sorted_pairs")
    assert_equal(host(out["pair_pos"]), ref["pair_pos"], "pair_pos")
    nt = int(host(out["n_tiles"])[0])
    assert nt == ref["n_tiles"]
    assert_equal(host(out["tiles"])[:nt], ref["tiles"], "tiles")
    assert int(host(out["n_dropped"])[0]) == ref["n_dropped"]


@pytest.mark.parametrize("T,topk,E,ns,bm,seed", [
    (1, 8, 384, 1, 16, 1), (8, 8, 384, 1, 16, 2), (64, 8, 384, 1, 16, 3),
    (113, 8, 384, 1, 16, 4),            # 1017 pairs: single-launch path
    (20, 8, 2000, 1, 16, 10),           # more experts than the histogram form holds
    (114, 8, 384, 1, 16, 5),            # 1026 pairs: three-kernel path
    (3000, 8, 384, 1, 64, 6), (2048, 8, 384, 0, 256, 7), (16, 2, 8, 0, 16, 8),
    (500, 4, 4000, 2, 32, 9),
    (5000, 8, 384, 1, 16, 13), (8192, 8, 384, 1, 192, 12)])   # 44 / 72 chunks: batched chunk scan
def test_permute_parity(gpu_lib, T, topk, E, ns, bm, seed):
    g = np.random.default_rng(seed)
    ids = np.stack([g.permutation(E)[:topk] for _ in range(T)]).astype(np.int32)
    _perm_check(gpu_lib, ids, E, ns, bm)


def test_permute_dropped_and_skewed(gpu_lib):
    g = np.random.default_rng(11)
    for T in (50, 400):
        ids = g.integers(-3, 390, size=(T, 8)).astype(np.int32)   # duplicates and invalid ids
        _perm_check(gpu_lib, ids, 384, 1, 16)
        ids = np.zeros((T, 8), dtype=np.int32)                     # everything on expert 0
        _perm_check(gpu_lib, ids, 384, 1, 16)


def test_permute_empty(gpu_lib):
    out = gpu_lib.moe_permute(torch.zeros((0, 8), dtype=torch.int32, device="cuda"), 384, 1, 16)
    assert int(host(out["n_tiles"])[0]) == 0
    assert np.all(host(out["expert_offsets"]) == 0)


# ------------------------------------------------------------------ fused routing + permutation

@pytest.mark.parametrize("T,E,ng,tg,topk,ns,bm,bstd,seed", [
    (1, 384, 8, 4, 8, 1, 16, 0.1, 21), (8, 384, 8, 4, 8, 1, 16, 0.1, 22),
    (64, 384, 8, 4, 8, 1, 16, 0.1, 23), (113, 384, 8, 4, 8, 1, 16, 0.1, 24),
    (16, 8, 1, 1, 2, 0, 16, 0.1, 25), (20, 120, 5, 2, 6, 2, 64, 0.5, 26),
    (0, 384, 8, 4, 8, 1, 16, 0.1, 27),
    (100, 1024, 16, 2, 8, 1, 16, 0.5, 28),   # 900 pairs over 8 wavefronts (E > 512)
    (40, 384, 2, 1, 8, 1, 32, 0.1, 29), (70, 384, 4, 2, 8, 0, 64, 0.0, 30),
    (9, 320, 8, 4, 8, 3, 1, 0.1, 31)])
def test_route_permute_fused(gpu_lib, T, E, ng, tg, topk, ns, bm, bstd, seed):
    """One launch gives what moe_route then moe_permute give, and the oracle."""
    g = np.random.default_rng(seed)
    logits = g.standard_normal((T, E), dtype=np.float32)
    bias = (g.standard_normal(E, dtype=np.float32) * np.float32(bstd)).astype(np.float32)
    ids, w, perm = gpu_lib.moe_route_permute(dev(logits), dev(bias), ng, tg, topk, ns, bm)
    rid, rw = OR.moe_route(logits, bias, ng, tg, topk)
    assert_equal(host(ids), rid.reshape(T, topk), "topk_ids")
    np.testing.assert_allclose(host(w), rw.reshape(T, topk), rtol=1e-6, atol=0)
    ref = OP.moe_permute(rid.reshape(T, topk).astype(np.int32), E, ns, bm)
    for name in ("expert_offsets", "sorted_pairs", "pair_pos"):
        assert_equal(host(perm[name]), ref[name], name)
    nt = int(host(perm["n_tiles"])[0])
    assert nt == ref["n_tiles"]
    assert_equal(host(perm["tiles"])[:nt], ref["tiles"], "tiles")
    assert int(host(perm["n_dropped"])[0]) == ref["n_dropped"]
    if T:
        # and bit for bit what the two separate calls write
        ids2, w2 = gpu_lib.moe_route(dev(logits), dev(bias), ng, tg, topk)
        perm2 = gpu_lib.moe_permute(ids2, E, ns, bm)
        assert_equal(host(w), host(w2), "weights vs moe_route")
        for name in ("expert_offsets", "sorted_pairs", "pair_pos"):
            assert_equal(host(perm[name]), host(perm2[name]), name + " vs moe_permute")


def test_route_permute_fused_ties(gpu_lib):
    """Coarse logits: many equal keys inside and across groups, several tokens
    per wavefront."""
    g = np.random.default_rng(32)
    T, E = 100, 384
    logits = (np.round(g.standard_normal((T, E)) * 2) / 2).astype(np.float32)
    bias = np.zeros(E, dtype=np.float32)
    ids, w, perm = gpu_lib.moe_route_permute(dev(logits), dev(bias), 8, 4, 8, 1, 16)
    rid, rw = OR.moe_route(logits, bias, 8, 4, 8)
    assert_equal(host(ids), rid.reshape(T, 8), "topk_ids")
    np.testing.assert_allclose(host(w), rw.reshape(T, 8), rtol=1e-6, atol=0)
    ref = OP.moe_permute(rid.reshape(T, 8).astype(np.int32), E, 1, 16)
    for name in ("expert_offsets", "sorted_pairs", "pair_pos"):
        assert_equal(host(perm[name]), ref[name], name)
    nt = int(host(perm["n_tiles"])[0])
    assert nt == ref["n_tiles"]
    assert_equal(host(perm["tiles"])[:nt], ref["tiles"], "tiles")


# ------------------------------------------------------------------ MXFP4 quant

def _quant_inputs(seed, M, K):
    g = np.random.default_rng(seed)
    x = g.standard_normal((M, K)).astype(np.float32) * np.exp(g.uniform(-8, 8, (M, 1))).astype(np.float32)
    xb = synth.bf16_from_f32(x)
    # edge rows: zeros, -0, bf16 subnormals, largest finite, exact E2M1 tie points
    xb[0, :] = 0
    xb[1, :32] = 0x8000
    xb[2, :] = np.arange(K, dtype=np.uint16) % 128 + 1            # subnormal bf16
    xb[3, :32] = 0x7f7f                                          # largest finite bf16
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 7.5, -0.25, -5.0], np.float32)
    xb[4, :12] = synth.bf16_from_f32(ties)
    xb[4, 12:32] = synth.bf16_from_f32(np.full(20, 0.1, np.float32))
    return xb


@pytest.mark.parametrize("M,K", [(16, 256), (37, 7168), (300, 2048), (9, 800), (6, 96)])
def test_mxfp4_quant_parity(gpu_lib, M, K):
    xb = _quant_inputs(M + K, M, K)
    codes, scales = gpu_lib.mxfp4_quant_1x32(bf16_dev(xb))
    rc, rs = OQ.mxfp4_quant_1x32(xb)
    assert_equal(host(scales), rs, "scales")
    assert_equal(host(codes), rc, "codes")


def test_mxfp4_quant_gather_and_row_count(gpu_lib):
    xb = _quant_inputs(5, 40, 512)
    gather = np.random.default_rng(6).integers(0, 40, 70).astype(np.int32)
    codes = torch.full((70, 256), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((70, 16), 0xCD, dtype=torch.uint8, device="cuda")
    rc_dev = dev(np.array([51], dtype=np.int32))
    gpu_lib.mxfp4_quant_1x32(bf16_dev(xb), row_gather=dev(gather), row_count=rc_dev,
                             codes=codes, scales=scales)
    rc, rs = OQ.mxfp4_quant_1x32(xb[gather])
    assert_equal(host(codes)[:51], rc[:51], "gathered codes")
    assert_equal(host(scales)[:51], rs[:51], "gathered scales")
    assert np.all(host(codes)[51:] == 0xAB) and np.all(host(scales)[51:] == 0xCD)


def chunk_major(codes, scales):
    """Row-major MXFP4 codes [M, K/2] / scales [M, K/32] in the chunk-major
    layout: codes [K/128, M, 64], scales [K/128, M, 4] (an index permutation)."""
    M, kb = codes.shape
    return (np.ascontiguousarray(codes.reshape(M, kb // 64, 64).transpose(1, 0, 2)),
            np.ascontiguousarray(scales.reshape(M, kb // 64, 4).transpose(1, 0, 2)))


def test_mxfp4_quant_every_finite_bf16(gpu_lib):
    """Every finite bf16 pattern goes through the quantizer (the E2M1 codes come
    from the hardware conversion): sorted by magnitude, so that each block holds
    neighbouring values and the codes span the grid, and in a seeded shuffle."""
    pats = np.arange(65536, dtype=np.uint32)
    finite = pats[(pats & 0x7F80) != 0x7F80].astype(np.uint16)
    n = (finite.size // 256) * 256
    order = np.argsort(finite & 0x7FFF, kind="stable")
    for xb in (finite[order][:n], np.random.default_rng(5).permutation(finite)[:n]):
        xb = xb.reshape(-1, 256)
        codes, scales = gpu_lib.mxfp4_quant_1x32(bf16_dev(xb))
        rc, rs = OQ.mxfp4_quant_1x32(xb)
        assert_equal(host(scales), rs, "scales")
        assert_equal(host(codes), rc, "codes")


@pytest.mark.parametrize("M,K", [(8, 128), (37, 512), (64, 7168), (5, 640)])
def test_mxfp4_quant_chunked_parity(gpu_lib, M, K):
    xb = _quant_inputs(M * 3 + K, M, K)
    codes, scales = gpu_lib.mxfp4_quant_1x32_chunked(bf16_dev(xb))
    rc, rs = chunk_major(*OQ.mxfp4_quant_1x32(xb))
    assert_equal(host(scales), rs, "chunked scales")
    assert_equal(host(codes), rc, "chunked codes")


def test_mxfp4_quant_chunked_scatter_and_row_count(gpu_lib):
    xb = _quant_inputs(9, 30, 256)
    k = 3
    g = np.random.default_rng(8)
    pos = g.permutation(30 * k).astype(np.int32)          # pair (t, j) -> sorted row
    pos[g.choice(30 * k, 7, replace=False)] = -1           # dropped pairs
    pos[5] = 10**6                                         # out of range: skipped
    codes = torch.full((2, 90, 64), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((2, 90, 4), 0xCD, dtype=torch.uint8, device="cuda")
    gpu_lib.mxfp4_quant_1x32_chunked(bf16_dev(xb), row_map=dev(pos), map_k=k, codes=codes,
                                     scales=scales)
    rc, rs = chunk_major(*OQ.mxfp4_quant_1x32(xb))
    hc, hs = host(codes), host(scales)
    written = np.zeros(90, bool)
    for p_, o in enumerate(pos):
        if 0 <= o < 90:
            written[o] = True
            assert_equal(hc[:, o], rc[:, p_ // k], f"row {o}")
            assert_equal(hs[:, o], rs[:, p_ // k], f"scale row {o}")
    assert np.all(hc[:, ~written] == 0xAB) and np.all(hs[:, ~written] == 0xCD)
    # row_count limits the input rows without a map
    codes2, scales2 = gpu_lib.mxfp4_quant_1x32_chunked(
        bf16_dev(xb), row_count=dev(np.array([11], np.int32)),
        codes=torch.full((2, 30, 64), 0xAB, dtype=torch.uint8, device="cuda"),
        scales=torch.full((2, 30, 4), 0xCD, dtype=torch.uint8, device="cuda"))
    assert_equal(host(codes2)[:, :11], rc[:, :11], "row_count codes")
    assert np.all(host(codes2)[:, 11:] == 0xAB) and np.all(host(scales2)[:, 11:] == 0xCD)


# ------------------------------------------------------------------ NVFP4 QDQ

@pytest.mark.parametrize("M,K,static", [(16, 256, False), (64, 7168, False), (33, 2048, True)])
def test_nvfp4_qdq_parity(gpu_lib, M, K, static):
    g = np.random.default_rng(M * K)
    xb = synth.bf16_from_f32(g.standard_normal((M, K)).astype(np.float32) *
                             np.exp(g.uniform(-3, 3, (M, 1))).astype(np.float32))
    xb[1, :16] = 0
    ts = np.float32(0.0037) if static else None
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((M, K // 16), dtype=torch.uint8, device="cuda")
    tso = torch.empty(1, dtype=torch.float32, device="cuda")
    y = gpu_lib.nvfp4_qdq(bf16_dev(xb), tensor_scale=None if ts is None else dev(np.array([ts])),
                          codes=codes, scales=scales, tensor_scale_out=tso)
    ref = OQ.nvfp4_qdq(xb, tensor_scale_in=ts)
    assert host(tso)[0] == np.float32(ref["tensor_scale"])
    assert_equal(host(scales), ref["scales"], "e4m3 scales")
    assert_equal(host(codes), ref["codes"], "codes")
    assert_equal(bits_of(y), ref["y"], "y")


def _pow2_below(s_t):
    """2^p <= s_t < 2^(p+1) for a normal float32 s_t (2^-126 for zero / subnormal)."""
    bits = np.array([s_t], np.float32).view(np.uint32)[0] & np.uint32(0x7F800000)
    return np.array([max(bits, 0x00800000)], np.uint32).view(np.float32)[0]


@pytest.mark.parametrize("M,K,ts", [(64, 7168, None), (33, 2048, 0.0037), (16, 256, 2.0 ** -120),
                                    (16, 256, 3.0e5), (24, 512, 2.0 ** -130)])
def test_nvfp4_qdq_f16_form(gpu_lib, M, K, ts):
    """The f16 operand form: y_f16 * y_f16_scale equals the oracle's y exactly,
    for dynamic, tiny, large and subnormal tensor scales."""
    g = np.random.default_rng(M + K)
    xb = synth.bf16_from_f32(g.standard_normal((M, K)).astype(np.float32) *
                             np.exp(g.uniform(-3, 3, (M, 1))).astype(np.float32))
    if ts is not None and ts < 1e-30:
        xb = synth.bf16_from_f32(F.bf16_decode(xb).astype(np.float32) * np.float32(ts * 1e3))
    xb[1, :16] = 0
    xb[2, :16] = 0x8000
    tsd = None if ts is None else dev(np.array([ts], np.float32))
    ref = OQ.nvfp4_qdq(xb, tensor_scale_in=None if ts is None else np.float32(ts))
    p2 = _pow2_below(np.float32(ref["tensor_scale"]))
    y16 = torch.full((M, K), float("nan"), dtype=torch.float16, device="cuda")
    sc = torch.zeros(1, dtype=torch.float32, device="cuda")
    y = gpu_lib.nvfp4_qdq(bf16_dev(xb), tensor_scale=tsd, y_f16=y16, y_f16_scale=sc)
    assert_equal(bits_of(y), ref["y"], "y")
    assert host(sc)[0] == p2
    want = F.bf16_decode(ref["y"])
    got = host(y16).astype(np.float64) * np.float64(p2)
    assert np.array_equal(got, want), "y_f16 * scale != y"
    assert np.array_equal(np.signbit(host(y16)), np.signbit(want)), "signs of zeros"
    # without the bf16 output
    y16b = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    none = gpu_lib.nvfp4_qdq(bf16_dev(xb), tensor_scale=tsd, y_f16=y16b, y_f16_scale=sc,
                             no_y=True)
    assert none is None
    assert np.array_equal(host(y16b).view(np.uint16), host(y16).view(np.uint16))


def test_nvfp4_qdq_row_count_and_zero(gpu_lib):
    g = np.random.default_rng(3)
    xb = synth.bf16_from_f32(g.standard_normal((20, 64)).astype(np.float32))
    xb[12:] = synth.bf16_from_f32(np.full((8, 64), 1e4, np.float32))   # must not enter amax
    y = gpu_lib.nvfp4_qdq(bf16_dev(xb), row_count=dev(np.array([12], np.int32)))
    ref = OQ.nvfp4_qdq(xb[:12])
    assert_equal(bits_of(y)[:12], ref["y"], "y rows < row_count")
    y0 = gpu_lib.nvfp4_qdq(bf16_dev(np.zeros((4, 32), np.uint16)))
    assert np.all(bits_of(y0) == 0)


# ------------------------------------------------------------------ FP8 conversion

def _convert_check(gpu_lib, codes, scales):
    fp8, sc, st, ni = gpu_lib.mxfp4_to_fp8_channel(dev(codes), dev(scales))
    ref = OC.mxfp4_to_fp8_channel(codes, scales)
    assert_equal(host(fp8), ref["fp8"], "fp8 codes")
    assert_equal(host(sc), ref["scale"], "channel scale")
    assert_equal(host(st), ref["status"], "row status")
    assert int(host(ni)[0]) == ref["n_inexact"]


def test_convert_golden_rows(gpu_lib):
    cases = load_convert_golden()
    codes = np.stack([c[1] for c in cases])
    scales = np.stack([c[2] for c in cases])
    _convert_check(gpu_lib, codes, scales)


@pytest.mark.parametrize("R,K,lo,hi,seed", [(512, 256, 0, 9, 1), (300, 7168, 1, 9, 2),
                                            (700, 2048, 1, 9, 3), (400, 512, 8, 20, 4),
                                            (64, 4096, 0, 40, 5), (12, 16384, 1, 9, 6),
                                            (10, 32768, 1, 12, 7)])
def test_convert_parity(gpu_lib, R, K, lo, hi, seed):
    g = np.random.default_rng(seed)
    codes = g.integers(0, 256, (R, K // 2), dtype=np.uint8)
    scales, _ = synth.spanned_scales(R, K // 32, 5, seed, top_lo=-4, top_hi=0, span_lo=lo,
                                     span_hi=hi)
    # sprinkle NaN blocks, zero rows and extreme scale rows
    scales[3, 1] = 255
    codes[5] = 0
    codes[6] = 0x88
    scales[7] = 254
    scales[8] = 0
    _convert_check(gpu_lib, codes, scales)


def test_convert_full_size_sampled(gpu_lib):
    """The conversion at the benchmarked size (the gate/up weights of all 385
    experts, 1576960 rows x 7168, row scale spans U{1..9} binades): every row
    exact (status 0, no inexact row: the span <= 9 invariant at full size), and
    sampled rows bit-exact against the oracle."""
    w = synth.WORKLOADS["skewed"]
    R, K = (w.E + w.n_shared) * 2 * w.I, w.H
    g = np.random.default_rng(99)
    codes = g.integers(0, 256, (R, K // 2), dtype=np.uint8)
    scales, _ = synth.spanned_scales(R, K // 32, 5, 99, top_lo=-4, top_hi=0, span_lo=1, span_hi=9)
    fp8, sc, st, ni = gpu_lib.mxfp4_to_fp8_channel(dev(codes), dev(scales))
    assert int(host(ni)[0]) == 0
    assert not np.any(host(st))
    rows = np.unique(np.concatenate([[0, 1, R // 2, R - 1], g.choice(R, 60, replace=False)]))
    ref = OC.mxfp4_to_fp8_channel(codes[rows], scales[rows])
    assert_equal(host(fp8[rows]), ref["fp8"], "fp8 codes (sampled rows)")
    assert_equal(host(sc[rows]), ref["scale"], "channel scale (sampled rows)")
    assert_equal(host(st[rows]), ref["status"], "row status (sampled rows)")
    del fp8, sc, st
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ combine

@pytest.mark.parametrize("T,topk,ns,H", [(1, 8, 1, 7168), (37, 2, 0, 256), (300, 8, 1, 2048),
                                         (140000, 8, 1, 64)])  # grid rows stride over the tokens
def test_combine_parity(gpu_lib, T, topk, ns, H):
    g = np.random.default_rng(T * H)
    k = topk + ns
    y = synth.bf16_from_f32(g.standard_normal((T * k, H)).astype(np.float32) * 50)
    pos = g.permutation(T * k).astype(np.int32)
    pos[::17] = -1
    w = g.uniform(0, 1, (T, topk)).astype(np.float32)
    out_f32 = torch.empty((T, H), dtype=torch.float32, device="cuda")
    out = gpu_lib.moe_combine(bf16_dev(y), dev(pos), dev(w), topk, ns, out_f32=out_f32)
    ref, _ = OG.moe_combine(F.bf16_decode(y), pos, w.astype(np.float64), T, topk, ns)
    assert_bf16_close(bits_of(out), ref, "combine")
    assert_float_close(host(out_f32), ref, "combine f32", rel_l2=1e-6, max_abs_rms=1e-5)


# ------------------------------------------------------------------ FP8 per token

def _fp8_rows(host_codes):
    """chunk-major [K/128, rows, 128] -> row-major [rows, K]."""
    c = np.asarray(host_codes)
    return np.ascontiguousarray(c.transpose(1, 0, 2)).reshape(c.shape[1], -1)


@pytest.mark.parametrize("M,K", [(33, 128), (7, 7168), (300, 2048), (5, 8192)])
def test_fp8_quant_per_token_parity(gpu_lib, M, K):
    """Codes (chunk-major) and per-row scales bit-exact against the oracle, rows
    of magnitudes 2^-12 .. 2^12, a zero row and a row of negative zeros."""
    g = np.random.default_rng(M * K)
    x = g.standard_normal((M, K)).astype(np.float32) * np.exp2(g.uniform(-12, 12, (M, 1))).astype(np.float32)
    x[0] = 0.0
    if M > 1:
        x[1] = -0.0
    xb = synth.bf16_from_f32(x)
    codes, scales = gpu_lib.fp8_quant_per_token(bf16_dev(xb))
    rc, rs = OQ.fp8_quant_per_token(xb)
    assert_equal(_fp8_rows(host(codes)), rc, "fp8 codes")
    assert_equal(host(scales), rs, "fp8 row scales")


def test_fp8_quant_every_finite_bf16(gpu_lib):
    """Every finite bf16 pattern (non-finite ones replaced by zero), 32 rows of
    2048, through the GPU quantizer and the oracle: bit-exact codes and scales
    (the division and the E4M3 rounding, ties and subnormals included)."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = (pats & 0x7F80) != 0x7F80
    xb = np.where(finite, pats, 0).astype(np.uint16).reshape(32, 2048)
    codes, scales = gpu_lib.fp8_quant_per_token(bf16_dev(xb))
    rc, rs = OQ.fp8_quant_per_token(xb)
    assert_equal(_fp8_rows(host(codes)), rc, "fp8 codes, every finite bf16")
    assert_equal(host(scales), rs, "fp8 row scales, every finite bf16")


def test_fp8_quant_row_count_and_slab(gpu_lib):
    """Rows at or past the device row count are not written; the output slab
    may be taller than M."""
    M, K, out_rows = 40, 256, 48
    g = np.random.default_rng(5)
    xb = synth.bf16_from_f32(g.standard_normal((M, K)).astype(np.float32))
    codes = torch.full((K // 128, out_rows, 128), 0xEE, dtype=torch.uint8, device="cuda")
    scales = torch.full((out_rows,), -1.0, dtype=torch.float32, device="cuda")
    gpu_lib.fp8_quant_per_token(bf16_dev(xb), row_count=dev(np.array([29], np.int32)),
                                out_rows=out_rows, codes=codes, scales=scales)
    rc, rs = OQ.fp8_quant_per_token(xb[:29])
    hc, hs = _fp8_rows(host(codes)), host(scales)
    assert_equal(hc[:29], rc, "codes of the counted rows")
    assert_equal(hs[:29], rs, "scales of the counted rows")
    assert np.all(hc[29:] == 0xEE) and np.all(hs[29:] == -1.0), "rows past the count"
