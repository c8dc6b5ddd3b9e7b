"""GPU parity of fp4_grouped_gemm (both stages, every supported format pair).

Each stage is checked on its own synthetic inputs (stage 2 gets a synthetic h,
never the GPU's stage-1 output), so the expected values come from the oracle
alone.  Shapes span several tiles per expert with ragged tails, a shared
expert, empty experts, and the full 7168/2048 layer width.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import gemm as OG
from oracle import permute as OP
from oracle import quant as OQ

from .parity import assert_bf16_close, assert_equal, assert_float_close
from .test_gpu_kernels import bf16_dev, bits_of, chunk_major, dev, host

pytestmark = pytest.mark.gpu


def make_weights(rng, Et, N, K, wfmt, lo=-6, hi=0):
    """Synthetic weights of one projection: dict(codes, scale[, ts]) as numpy."""
    if wfmt == "mx":
        return dict(codes=rng.integers(0, 256, (Et, N, K // 2), dtype=np.uint8),
                    scale=(127 + rng.integers(lo, hi + 1, (Et, N, K // 32))).astype(np.uint8))
    if wfmt == "nvfp4":
        return dict(codes=rng.integers(0, 256, (Et, N, K // 2), dtype=np.uint8),
                    scale=synth.e4m3_from_f32(np.abs(rng.standard_normal((Et, N, K // 16),
                                                                         dtype=np.float32))),
                    ts=rng.uniform(0.01, 0.02, Et).astype(np.float32))
    if wfmt == "fp8":
        c = rng.integers(0, 256, (Et, N, K), dtype=np.uint8)
        c[(c & 0x7F) == 0x7F] = 0x3C
        return dict(codes=c, scale=np.ldexp(1.0, rng.integers(-9, -3, (Et, N))).astype(np.float32))
    raise ValueError(wfmt)


def oracle_weight(wd, wfmt, e):
    if wfmt == "nvfp4":
        return OG.dequant_expert(wfmt, wd["codes"][e], wd["scale"][e], wd["ts"][e])
    return OG.dequant_expert(wfmt, wd["codes"][e], wd["scale"][e])


def gpu_weight_args(wd, wfmt):
    kw = dict(w=dev(wd["codes"]))
    if wfmt == "fp8":
        kw.update(w_scale=None, w_channel_scale=dev(wd["scale"]))
    else:
        kw.update(w_scale=dev(wd["scale"]))
    if wfmt == "nvfp4":
        kw.update(w_tensor_scale=dev(wd["ts"]))
    return kw


def routing(rng, T, topk, E, skew=False):
    if skew:
        p = 1.0 / np.arange(1, E + 1) ** 1.5
        p /= p.sum()
        return np.stack([rng.choice(E, topk, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    return np.stack([rng.permutation(E)[:topk] for _ in range(T)]).astype(np.int32)


def run_stage(gpu_lib, stage, wfmt, afmt, T, topk, E, ns, H, I, bm, seed, skew=False,
              exact=False, layout=0, a_layout=0, with_f32=True, quant_out=False, ids=None):
    rng = np.random.default_rng(seed)
    Et = E + ns
    k = topk + ns
    if ids is None:
        ids = routing(rng, T, topk, E, skew)
    perm_ref = OP.moe_permute(ids, E, ns, bm)
    perm = gpu_lib.moe_permute(dev(ids), E, ns, bm)
    n_rows = int(perm_ref["expert_offsets"][-1])
    N, K = (2 * I, H) if stage == 1 else (H, I)
    if exact:
        wd = dict(codes=rng.integers(0, 256, (Et, N, K // 2), dtype=np.uint8),
                  scale=np.full((Et, N, K // 32), 127, np.uint8))
        vals = np.array([0, .5, 1, 1.5, 2, -.5, -1, -1.5, -2], np.float32)
    else:
        wd = make_weights(rng, Et, N, K, wfmt)
    # activations: stage 1 reads token rows through the gather, stage 2 sorted rows
    rows_in = T if stage == 1 else T * k
    if exact:
        xf = vals[rng.integers(0, len(vals), (rows_in, K))]
    else:
        xf = rng.standard_normal((rows_in, K), dtype=np.float32) * np.float32(1 if stage == 1 else 20)
    xb = synth.bf16_from_f32(xf)
    poison = stage == 2 and n_rows < rows_in     # rows past the valid count are never read
    if afmt == "mx":
        qc, qs = OQ.mxfp4_quant_1x32(xb)
        a_vals = F.mxfp4_dequant(qc, qs)
        if poison:
            qs = qs.copy()
            qs[n_rows:] = 255
        a_kw = dict(a=dev(qc), a_scale=dev(qs), afmt=gpu_lib.A_MXFP4)
    elif afmt == "fp8":
        # per-token FP8 from the oracle's quantizer, chunk-major; rows past the
        # valid count poisoned (NaN codes, NaN scales) for stage 2
        codes, sc = OQ.fp8_quant_per_token(xb)
        a_vals = F.e4m3_decode(codes) * sc.astype(np.float64)[:, None]
        if poison:
            codes, sc = codes.copy(), sc.copy()
            codes[n_rows:] = 0x7F
            sc[n_rows:] = np.nan
        cm = np.ascontiguousarray(codes.reshape(rows_in, K // 128, 128).transpose(1, 0, 2))
        a_kw = dict(a=dev(cm), a_row_scale=dev(sc), afmt=gpu_lib.A_FP8)
    elif afmt == "f16":
        # NVFP4 activations in the f16 operand form, made on the host from the
        # oracle's QDQ: y * 2^-p is exact in f16
        r = OQ.nvfp4_qdq(xb)
        s_t = np.float32(r["tensor_scale"])
        bits = np.array([s_t], np.float32).view(np.uint32)[0] & np.uint32(0x7F800000)
        p2 = np.array([bits], np.uint32).view(np.float32)[0]
        a_vals = F.bf16_decode(r["y"])
        a16 = (a_vals / np.float64(p2)).astype(np.float16)
        assert np.array_equal(a16.astype(np.float64) * np.float64(p2), a_vals)
        if poison:
            a16 = a16.copy()
            a16[n_rows:] = np.float16("nan")
        a_kw = dict(a=dev(a16.view(np.int16)).view(torch.float16), afmt=gpu_lib.A_F16,
                    a_f16_scale=dev(np.array([p2], np.float32)))
    else:
        a_vals = F.bf16_decode(xb)
        if poison:
            xb = xb.copy()
            xb[n_rows:] = 0x7FC0
        a_kw = dict(a=bf16_dev(xb), afmt=gpu_lib.A_BF16)
    if stage == 1:
        a_sorted = a_vals[perm_ref["sorted_pairs"][:n_rows] // k]
        gather = dict(a_row_gather=perm["sorted_pairs"], gather_div=k)
    else:
        a_sorted = a_vals[:n_rows]
        gather = {}
    if a_layout == 1 and afmt == "mx":
        # chunk-major activations, already in expert order (stage 1: gathered
        # here, on the host), rows past the valid count poisoned
        rows = T * k
        if stage == 1:
            src = np.zeros(rows, np.int64)
            src[:n_rows] = perm_ref["sorted_pairs"][:n_rows] // k
            qc, qs = qc[src], qs[src].copy()
            qs[n_rows:] = 255
        cc, cs = chunk_major(qc, qs)
        a_kw = dict(a=dev(cc), a_scale=dev(cs), afmt=gpu_lib.A_MXFP4)
        gather = {}
    n_out = N // 2 if stage == 1 else N
    out_f32 = (torch.full((T * k, n_out), float("nan"), dtype=torch.float32, device="cuda")
               if with_f32 else None)
    afmt_code = a_kw.pop("afmt")
    wkw = gpu_weight_args(wd, wfmt)
    if layout == gpu_lib.LAYOUT_FRAGMENT:
        c, sc = gpu_lib.fp4_weight_preshuffle(gpu_lib.WFMT[wfmt], wkw["w"], wkw["w_scale"])
        wkw["w"] = c
        if wfmt != "fp8":
            wkw["w_scale"] = sc
    qkw = {}
    if quant_out:
        # stage-1 output also quantized in the epilogue; unwritten bytes stay 0xEE
        rows = T * k
        qkw = dict(out_q=torch.full((n_out // 128, rows, 64), 0xEE, dtype=torch.uint8, device="cuda"),
                   out_q_scale=torch.full((n_out // 128, rows, 4), 0xEE, dtype=torch.uint8,
                                          device="cuda"))
    out = gpu_lib.fp4_grouped_gemm(stage, gpu_lib.WFMT[wfmt], afmt_code,
                                   perm=perm, block_m=bm, out_f32=out_f32, w_layout=layout,
                                   a_layout=a_layout, **wkw, **a_kw, **gather, **qkw)
    if quant_out:
        # the codes are mxfp4_quant_1x32 of the bf16 output rows, in the
        # chunk-major layout; rows past the valid count are not written
        h_bits = bits_of(out)[:n_rows]
        rc, rs = OQ.mxfp4_quant_1x32(h_bits)
        cc, cs = chunk_major(rc, rs)
        gq, gs = host(qkw["out_q"]), host(qkw["out_q_scale"])
        assert np.array_equal(gq[:, :n_rows], cc), "quantized h codes"
        assert np.array_equal(gs[:, :n_rows], cs), "quantized h scales"
        assert np.all(gq[:, n_rows:] == 0xEE) and np.all(gs[:, n_rows:] == 0xEE), "rows past the end"
        # and the same bytes when the bf16 output is not written at all
        q2 = dict(out_q=torch.zeros_like(qkw["out_q"]), out_q_scale=torch.zeros_like(qkw["out_q_scale"]))
        none = gpu_lib.fp4_grouped_gemm(stage, gpu_lib.WFMT[wfmt], afmt_code, perm=perm, block_m=bm,
                                        w_layout=layout, a_layout=a_layout, no_out=True, **wkw,
                                        **a_kw, **gather, **q2)
        assert none is None
        assert np.array_equal(host(q2["out_q"])[:, :n_rows], cc), "quantized h codes, no bf16 out"
        assert np.array_equal(host(q2["out_q_scale"])[:, :n_rows], cs), "scales, no bf16 out"
    ref_unrounded = OG.grouped_stage(stage, a_sorted, perm_ref["expert_offsets"],
                                     lambda e: oracle_weight(wd, wfmt, e), rounding=False)
    g_bits = bits_of(out)[:n_rows]
    if not with_f32:
        assert_bf16_close(g_bits, ref_unrounded, f"stage{stage} {wfmt}/{afmt} bf16 only")
        return
    g_f32 = host(out_f32)[:n_rows]
    if exact:
        assert np.array_equal(g_f32.astype(np.float64), ref_unrounded), "exact special case"
        return
    assert_float_close(g_f32, ref_unrounded, f"stage{stage} {wfmt}/{afmt} f32")
    assert_bf16_close(g_bits, ref_unrounded, f"stage{stage} {wfmt}/{afmt} bf16")


DQ_CASES = [
    # stage, wfmt, T, topk, E, ns, H, I, bm, seed, skew
    (1, "mx", 16, 2, 8, 0, 256, 128, 16, 1, False),
    (2, "mx", 16, 2, 8, 0, 256, 128, 16, 2, False),
    (1, "mx", 70, 3, 6, 1, 512, 256, 16, 3, True),
    (2, "mx", 70, 3, 6, 1, 512, 256, 16, 4, True),
    (1, "mx", 90, 4, 10, 1, 1024, 256, 32, 5, True),
    (2, "mx", 90, 4, 10, 1, 1024, 256, 64, 6, True),
    (1, "mx", 3, 2, 4, 1, 7168, 2048, 16, 7, False),
    (2, "mx", 3, 2, 4, 1, 7168, 2048, 16, 8, False),
    (1, "nvfp4", 60, 4, 8, 0, 512, 256, 64, 9, True),
    (2, "nvfp4", 60, 4, 8, 0, 512, 256, 64, 10, True),
    (1, "nvfp4", 40, 2, 12, 0, 1024, 512, 16, 11, False),
    (1, "fp8", 50, 2, 6, 1, 512, 256, 16, 12, True),
    (2, "fp8", 50, 2, 6, 1, 512, 256, 64, 13, True),
]


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("case", DQ_CASES)
def test_dq_gemm_parity(gpu_lib, case, layout):
    stage, wfmt, T, topk, E, ns, H, I, bm, seed, skew = case
    run_stage(gpu_lib, stage, wfmt, "bf16", T, topk, E, ns, H, I, bm, seed, skew, layout=layout)


F16_CASES = [
    # stage, T, topk, E, ns, H, I, seed, skew: NVFP4 weights x f16 activations,
    # 64-row tiles (32x32 f16 MFMA): several tiles per expert with ragged
    # tails, a shared expert, empty experts, full width, narrow width (4 waves)
    (1, 60, 4, 8, 0, 512, 256, 61, True),
    (2, 60, 4, 8, 0, 512, 256, 62, True),
    (1, 150, 6, 10, 1, 1024, 512, 63, True),
    (2, 150, 6, 10, 1, 1024, 512, 64, True),
    (1, 9, 3, 5, 1, 7168, 2048, 65, False),
    (2, 9, 3, 5, 1, 7168, 2048, 66, False),
    (1, 40, 2, 6, 0, 256, 128, 67, False),
    (2, 40, 2, 6, 0, 256, 256, 68, False),
]


@pytest.mark.parametrize("case", F16_CASES)
def test_nvfp4_f16_activation_gemm(gpu_lib, case):
    stage, T, topk, E, ns, H, I, seed, skew = case
    run_stage(gpu_lib, stage, "nvfp4", "f16", T, topk, E, ns, H, I, 64, seed, skew,
              layout=gpu_lib.LAYOUT_FRAGMENT)


F16_128_CASES = [
    # stage, T, topk, E, ns, H, I, seed, skew: NVFP4 weights x f16 activations
    # in 128-row tiles (K a multiple of 512): hot experts of several tiles with
    # ragged tails, a shared expert, empty experts, full width, narrow width
    (1, 300, 4, 8, 0, 512, 512, 71, True),
    (2, 300, 4, 8, 0, 512, 512, 72, True),
    (1, 150, 6, 10, 1, 1024, 512, 73, True),
    (2, 150, 6, 10, 1, 1024, 512, 74, True),
    (1, 9, 3, 5, 1, 7168, 2048, 75, False),
    (2, 9, 3, 5, 1, 7168, 2048, 76, False),
    (1, 40, 2, 6, 0, 512, 128, 77, False),
    (2, 40, 2, 6, 0, 256, 512, 78, False),
]


@pytest.mark.parametrize("case", F16_128_CASES)
def test_nvfp4_f16_activation_gemm_128_row_tiles(gpu_lib, case):
    stage, T, topk, E, ns, H, I, seed, skew = case
    run_stage(gpu_lib, stage, "nvfp4", "f16", T, topk, E, ns, H, I, 128, seed, skew,
              layout=gpu_lib.LAYOUT_FRAGMENT)


@pytest.mark.parametrize("stage,E,topk,H,I,Ts", [
    (1, 12, 4, 1024, 512, (400, 90)),
    (2, 12, 4, 1024, 512, (400, 90)),
    # fewer items than the eight XCD groups the cost split serves (one or two
    # column blocks, a handful of tiles)
    (1, 6, 1, 512, 512, (3, 5, 1)),
    (2, 6, 1, 512, 512, (3, 5, 1)),
])
def test_nvfp4_f16_128_row_tiles_work_queue(gpu_lib, stage, E, topk, H, I, Ts):
    """With a work queue the workgroups take their items as they free up: the
    same bytes as the fixed share (every item is computed the same way), on
    calls in a row with different row counts, and the queue zero-filled after
    each call."""
    rng = np.random.default_rng(90 + stage + H)
    N, K = (2 * I, H) if stage == 1 else (H, I)
    wd = make_weights(rng, E, N, K, "nvfp4")
    wc, ws = gpu_lib.fp4_weight_preshuffle(gpu_lib.W_NVFP4, dev(wd["codes"]), dev(wd["scale"]))
    queue = torch.zeros(16, dtype=torch.int32, device="cuda")
    for T in Ts:
        ids = routing(rng, T, topk, E, skew=True)
        perm = gpu_lib.moe_permute(dev(ids), E, 0, 128)
        rows_in = T if stage == 1 else T * topk
        a16 = (rng.integers(-6, 7, (rows_in, K)) * 0.25).astype(np.float16)
        a = dev(a16.view(np.int16)).view(torch.float16)
        kw = dict(a_f16_scale=dev(np.array([1.0], np.float32)), w_tensor_scale=dev(wd["ts"]),
                  w_layout=gpu_lib.LAYOUT_FRAGMENT)
        if stage == 1:
            kw.update(a_row_gather=perm["sorted_pairs"], gather_div=topk)
        outs = []
        for q in (None, queue):
            # rows never written would keep this pattern (a NaN in bf16)
            o = torch.full((T * topk, N // 2 if stage == 1 else N), -1, dtype=torch.int16,
                           device="cuda").view(torch.bfloat16)
            gpu_lib.fp4_grouped_gemm(stage, gpu_lib.W_NVFP4, gpu_lib.A_F16, wc, ws, a, perm,
                                     128, work_queue=q, out=o, **kw)
            torch.cuda.synchronize()
            outs.append(bits_of(o)[: int(host(perm["expert_offsets"])[-1])].copy())
            if q is not None:
                assert not host(q).any(), "queue left non-zero"
        assert not (outs[0] == 0xFFFF).any(), f"T={T}: rows left unwritten"
        assert outs[0].tobytes() == outs[1].tobytes(), f"T={T}: queue and fixed share differ"


@pytest.mark.parametrize("stage", [1, 2])
def test_nvfp4_f16_128_row_tiles_every_block_count(gpu_lib, stage):
    """Expert segments of 1, 33, 70, 127 and 225 rows: tiles with one, two,
    three and four live 32-row blocks, a full tile, and ragged ends of each."""
    counts = [1, 33, 70, 127, 225]
    ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    ids = np.random.default_rng(79).permutation(ids)[:, None].astype(np.int32)
    run_stage(gpu_lib, stage, "nvfp4", "f16", len(ids), 1, len(counts), 0, 512, 512, 128, 80 + stage,
              layout=gpu_lib.LAYOUT_FRAGMENT, ids=ids)


MX_CASES = [
    (1, "mx", 16, 2, 8, 0, 256, 128, 32, 21, False),
    (2, "mx", 16, 2, 8, 0, 256, 128, 32, 22, False),
    (1, "mx", 200, 3, 6, 1, 512, 256, 64, 23, True),
    (2, "mx", 200, 3, 6, 1, 512, 256, 64, 24, True),
    (1, "mx", 400, 4, 8, 1, 512, 256, 128, 25, True),
    (2, "mx", 400, 4, 8, 1, 512, 256, 256, 26, True),
    (1, "mx", 400, 4, 8, 1, 512, 256, 256, 33, True),
    (1, "mx", 300, 8, 8, 1, 1024, 512, 256, 34, False),
    (2, "mx", 300, 8, 8, 1, 1024, 512, 256, 35, False),
    (1, "mx", 300, 8, 8, 1, 1024, 512, 128, 36, False),
    (1, "mx", 5, 2, 4, 1, 7168, 2048, 32, 27, False),
    (2, "mx", 5, 2, 4, 1, 7168, 2048, 32, 28, False),
    (1, "fp8", 150, 3, 6, 1, 512, 256, 64, 29, True),
    (2, "fp8", 150, 3, 6, 1, 512, 256, 32, 30, True),
    (1, "fp8", 3, 2, 4, 1, 7168, 2048, 16, 32, False),
]

# block_m 192 (192 x 512 tiles, fragment-major weights only): experts of one
# and two M tiles, K of 1, 2 and several 128-wide chunks
WIDE_CASES = [
    (1, "mx", 400, 4, 8, 1, 512, 256, 192, 37, True),
    (2, "mx", 400, 4, 8, 1, 512, 256, 192, 38, True),
    (1, "mx", 300, 8, 8, 1, 1024, 512, 192, 39, False),
    (2, "mx", 300, 8, 8, 1, 1024, 512, 192, 40, False),
    (1, "mx", 100, 2, 4, 0, 128, 256, 192, 41, False),
    (2, "mx", 100, 2, 4, 0, 512, 128, 192, 42, False),
    # FP8 weights x MXFP4 activations on the scaled MFMA: 192 x 256 tiles
    (1, "fp8", 400, 4, 8, 1, 512, 256, 192, 43, True),
    (2, "fp8", 400, 4, 8, 1, 512, 256, 192, 44, True),
    (1, "fp8", 300, 8, 8, 1, 1024, 128, 192, 45, False),
    (2, "fp8", 100, 2, 4, 0, 256, 128, 192, 46, False),
    # more work items than workgroups (several items per workgroup, the FP8
    # tile prefetching the next item's first chunks), K of two chunks
    (1, "fp8", 1500, 8, 8, 1, 256, 512, 192, 47, True),
    (2, "fp8", 1500, 8, 8, 1, 1024, 256, 192, 48, True),
    (1, "mx", 1500, 8, 8, 1, 256, 1024, 192, 49, True),
    (2, "mx", 1500, 8, 8, 1, 2048, 256, 192, 50, True),
]


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("case", MX_CASES)
def test_mx_gemm_parity(gpu_lib, case, layout):
    stage, wfmt, T, topk, E, ns, H, I, bm, seed, skew = case
    run_stage(gpu_lib, stage, wfmt, "mx", T, topk, E, ns, H, I, bm, seed, skew, layout=layout)


@pytest.mark.parametrize("case", WIDE_CASES)
def test_mx_gemm_wide_tiles(gpu_lib, case):
    """192 x 512 tiles with row-major activations."""
    stage, wfmt, T, topk, E, ns, H, I, bm, seed, skew = case
    run_stage(gpu_lib, stage, wfmt, "mx", T, topk, E, ns, H, I, bm, seed, skew,
              layout=gpu_lib.LAYOUT_FRAGMENT)


@pytest.mark.parametrize("a_layout", [0, 1])
@pytest.mark.parametrize("case", WIDE_CASES)
def test_mx_gemm_wide_tiles_bf16_only(gpu_lib, case, a_layout):
    """Without the fp32 copy the 192 x 512 tiles write bf16 rows through LDS
    with 16-byte stores."""
    stage, wfmt, T, topk, E, ns, H, I, bm, seed, skew = case
    run_stage(gpu_lib, stage, wfmt, "mx", T, topk, E, ns, H, I, bm, seed, skew,
              layout=gpu_lib.LAYOUT_FRAGMENT, a_layout=a_layout, with_f32=False)


@pytest.mark.parametrize("a_layout", [0, 1])
@pytest.mark.parametrize("case", [c for c in WIDE_CASES if c[0] == 1])
def test_wide_stage1_quantized_output(gpu_lib, case, a_layout):
    """Stage 1 on 192-row tiles writes h also as chunk-major MXFP4, exactly
    what mxfp4_quant_1x32 makes of the bf16 h."""
    stage, wfmt, T, topk, E, ns, H, I, bm, seed, skew = case
    run_stage(gpu_lib, stage, wfmt, "mx", T, topk, E, ns, H, I, bm, seed, skew,
              layout=gpu_lib.LAYOUT_FRAGMENT, a_layout=a_layout, with_f32=False, quant_out=True)


@pytest.mark.parametrize("case", [c for c in MX_CASES if c[1] == "mx" and c[8] >= 128] + WIDE_CASES)
def test_mx_gemm_chunked_activations(gpu_lib, case):
    """Prefill tiles reading chunk-major, pre-gathered MXFP4 activations."""
    stage, wfmt, T, topk, E, ns, H, I, bm, seed, skew = case
    run_stage(gpu_lib, stage, wfmt, "mx", T, topk, E, ns, H, I, bm, seed, skew,
              layout=gpu_lib.LAYOUT_FRAGMENT, a_layout=gpu_lib.A_LAYOUT_CHUNKED)


@pytest.mark.parametrize("afmt,bm,layout", [("bf16", 16, 0), ("bf16", 64, 1), ("mx", 64, 0),
                                            ("mx", 256, 1)])
def test_gemm_exact_special_case(gpu_lib, afmt, bm, layout):
    """E8M0 = 127 weights and activations in {0, +-.5, +-1, +-1.5, +-2}: every
    product is a multiple of 0.25 below 12, every partial sum of K <= 4096 terms
    stays below 2^22 in quarter units, so the float32 stage-2 result is exact in
    any summation order and must equal the oracle bit for bit."""
    run_stage(gpu_lib, 2, "mx", afmt, 40, 2, 6, 1, 512, 2048, bm, 31, exact=True, layout=layout)


def _fragment_reference(codes, scales, wfmt):
    """Independent index-formula reference of the fragment-major layout."""
    E, N = codes.shape[:2]
    G = N // 16
    if wfmt == "fp8":
        K = codes.shape[2]
        C = K // 128
        e, n, k = np.meshgrid(np.arange(E), np.arange(N), np.arange(K), indexing="ij")
        lane = n % 16 + 16 * ((k % 128) // 32)
        f = (e * G + n // 16) * C + k // 128
        out = np.empty(codes.size, np.uint8)
        out[(f * 2048 + ((k % 32) // 16) * 1024 + lane * 16 + k % 16).ravel()] = codes.ravel()
        return out.reshape(codes.shape), None
    K = codes.shape[2] * 2
    C = K // 128
    e, n, kb = np.meshgrid(np.arange(E), np.arange(N), np.arange(K // 2), indexing="ij")
    lane = n % 16 + 16 * ((kb % 64) // 16)
    f = (e * G + n // 16) * C + kb // 64
    oc = np.empty(codes.size, np.uint8)
    oc[(f * 1024 + lane * 16 + kb % 16).ravel()] = codes.ravel()
    per = 1 if wfmt == "mx" else 2
    e, n, sb = np.meshgrid(np.arange(E), np.arange(N), np.arange(K // 32 * per), indexing="ij")
    blk = sb // per
    lane = n % 16 + 16 * (blk % 4)
    h = (e * C + blk // 4) * G + n // 16          # scales: chunk-major
    os_ = np.empty(scales.size, np.uint8)
    os_[(h * 64 * per + lane * per + sb % per).ravel()] = scales.ravel()
    return oc.reshape(codes.shape), os_.reshape(scales.shape)


@pytest.mark.parametrize("wfmt", ["mx", "nvfp4", "fp8"])
def test_preshuffle_layout(gpu_lib, wfmt):
    rng = np.random.default_rng(40)
    wd = make_weights(rng, 3, 48, 384, wfmt)
    codes_ref, scales_ref = _fragment_reference(wd["codes"], wd["scale"], wfmt)
    c, sc = gpu_lib.fp4_weight_preshuffle(gpu_lib.WFMT[wfmt], dev(wd["codes"]),
                                          None if wfmt == "fp8" else dev(wd["scale"]))
    assert np.array_equal(host(c), codes_ref)
    if wfmt != "fp8":
        assert np.array_equal(host(sc), scales_ref)


# ------------------------------------------------------------------ dense MXFP4 linear

LINEAR_CASES = [
    # M, N, K, a_layout, seed: single rows, ragged 192-row tails, several column
    # blocks, both activation layouts, the hidden width as K; the last two have
    # more row tiles than one group of the work order (8) and a short last group
    (1, 512, 128, 0, 81), (37, 512, 256, 1, 82), (192, 1024, 512, 0, 83),
    (500, 1536, 1024, 1, 84), (2000, 512, 7168, 0, 85), (385, 2048, 2048, 1, 86),
    (2000, 1536, 256, 1, 87), (3100, 2560, 384, 0, 88),
]


@pytest.mark.parametrize("case", LINEAR_CASES)
def test_mxfp4_linear_parity(gpu_lib, case):
    M, N, K, a_layout, seed = case
    rng = np.random.default_rng(seed)
    xb = synth.bf16_from_f32(rng.standard_normal((M, K), dtype=np.float32))
    qc, qs = OQ.mxfp4_quant_1x32(xb)
    a_vals = F.mxfp4_dequant(qc, qs)
    wd = make_weights(rng, 1, N, K, "mx")
    fc, fs = gpu_lib.fp4_weight_preshuffle(gpu_lib.WFMT["mx"], dev(wd["codes"]), dev(wd["scale"]))
    if a_layout == 1:
        rows = M + 5                     # a slab taller than M: rows past M are never read
        cpad = np.vstack([qc, np.full((rows - M, K // 2), 0x77, np.uint8)])
        spad = np.vstack([qs, np.full((rows - M, K // 32), 255, np.uint8)])
        cc, cs = chunk_major(cpad, spad)
        a, a_s = dev(cc), dev(cs)
    else:
        a, a_s = dev(qc), dev(qs)
    out_f32 = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    out = gpu_lib.mxfp4_linear(a, a_s, fc[0], fs[0], a_layout=a_layout, M=M, out_f32=out_f32)
    ref = OG.grouped_stage(2, a_vals, np.array([0, M]), lambda e: oracle_weight(wd, "mx", 0),
                           rounding=False)
    assert_float_close(host(out_f32), ref, "mxfp4_linear f32")
    assert_bf16_close(bits_of(out), ref, "mxfp4_linear bf16")


def test_mxfp4_linear_exact_special_case(gpu_lib):
    """E8M0 = 127 weights and activations on {0, +-.5, +-1, +-1.5, +-2}: every
    product and partial sum is exact, so the float32 output equals the oracle
    bit for bit."""
    rng = np.random.default_rng(87)
    M, N, K = 250, 1024, 2048
    vals = np.array([0, .5, 1, 1.5, 2, -.5, -1, -1.5, -2], np.float32)
    xb = synth.bf16_from_f32(vals[rng.integers(0, len(vals), (M, K))])
    qc, qs = OQ.mxfp4_quant_1x32(xb)
    codes = rng.integers(0, 256, (1, N, K // 2), dtype=np.uint8)
    scale = np.full((1, N, K // 32), 127, np.uint8)
    fc, fs = gpu_lib.fp4_weight_preshuffle(gpu_lib.WFMT["mx"], dev(codes), dev(scale))
    out_f32 = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    gpu_lib.mxfp4_linear(dev(qc), dev(qs), fc[0], fs[0], out_f32=out_f32)
    ref = F.mxfp4_dequant(qc, qs) @ OG.dequant_expert("mx", codes[0], scale[0]).T
    assert np.array_equal(host(out_f32).astype(np.float64), ref)


def test_mxfp4_linear_full_size_sampled(gpu_lib):
    """The dense linear at the benchmarked size and launch configuration (M=16384,
    N=K=7168, activations quantized chunk-major on the device, 192 x 512 tiles):
    the activation codes and the outputs of sampled rows (first and last rows,
    both sides of a 192-row tile boundary, random rows) against the oracle, for
    the float32-copy epilogue and for the bf16-only one the benchmark times."""
    M, N, K = 16384, 7168, 7168
    rng = np.random.default_rng(91)
    xb = synth.bf16_from_f32(rng.standard_normal((M, K), dtype=np.float32))
    wd = make_weights(rng, 1, N, K, "mx")
    fc, fs = gpu_lib.fp4_weight_preshuffle(gpu_lib.WFMT["mx"], dev(wd["codes"]), dev(wd["scale"]))
    codes, scales = gpu_lib.mxfp4_quant_1x32_chunked(bf16_dev(xb))
    out_f32 = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    out = gpu_lib.mxfp4_linear(codes, scales, fc[0], fs[0], a_layout=1, M=M, out_f32=out_f32)
    rows = np.unique(np.concatenate([[0, 191, 192, 8191, 8192, M - 1],
                                     rng.choice(M, 10, replace=False)]))
    qc, qs = OQ.mxfp4_quant_1x32(xb[rows])
    hc, hs = host(codes), host(scales)                 # [K/128, M, 64], [K/128, M, 4]
    assert_equal(np.ascontiguousarray(hc[:, rows].transpose(1, 0, 2)).reshape(len(rows), K // 2),
                 qc, "sampled activation codes")
    assert_equal(np.ascontiguousarray(hs[:, rows].transpose(1, 0, 2)).reshape(len(rows), K // 32),
                 qs, "sampled activation scales")
    ref = F.mxfp4_dequant(qc, qs) @ oracle_weight(wd, "mx", 0).T
    assert_float_close(host(out_f32)[rows], ref, "full-size mxfp4_linear f32 (sampled rows)")
    assert_bf16_close(bits_of(out)[rows], ref, "full-size mxfp4_linear bf16 (sampled rows)")
    # the launch the benchmark times: bf16 output only (the epilogue that goes
    # through LDS and leaves as 16-byte row stores)
    del out_f32
    out2 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    gpu_lib.mxfp4_linear(codes, scales, fc[0], fs[0], a_layout=1, M=M, out=out2)
    assert_bf16_close(bits_of(out2)[rows], ref, "full-size mxfp4_linear, bf16-only epilogue")
    assert not torch.isnan(out2).any().item(), "bf16-only epilogue left rows unwritten"


W8A8_CASES = [
    # stage, T, topk, E, ns, H, I, seed, skew: 128-row tiles, several per expert
    # with ragged tails, a shared expert, the full layer width
    (1, 300, 4, 8, 1, 512, 256, 60, False),
    (2, 300, 4, 8, 1, 512, 256, 61, False),
    (1, 600, 2, 5, 1, 512, 256, 62, True),
    (2, 600, 2, 5, 1, 1024, 256, 63, True),
    (1, 40, 8, 16, 1, 7168, 2048, 64, False),
    (2, 40, 8, 16, 1, 7168, 2048, 65, False),
]


@pytest.mark.parametrize("case", W8A8_CASES)
def test_w8a8_gemm_parity(gpu_lib, case):
    """FP8 weights (fragment-major, per-channel scales) x per-token FP8
    activations (chunk-major) on the scaled MFMA, 128-row tiles: float32 and
    bf16 outputs against the oracle on the same FP8 values."""
    stage, T, topk, E, ns, H, I, seed, skew = case
    run_stage(gpu_lib, stage, "fp8", "fp8", T, topk, E, ns, H, I, 128, seed, skew=skew,
              layout=gpu_lib.LAYOUT_FRAGMENT, a_layout=1)


def test_w8a8_gemm_bf16_only(gpu_lib):
    """The bf16-only epilogue (the one the layer runs) of the W8A8 tiles."""
    run_stage(gpu_lib, 2, "fp8", "fp8", 300, 4, 8, 1, 512, 256, 128, 66,
              layout=gpu_lib.LAYOUT_FRAGMENT, a_layout=1, with_f32=False)
