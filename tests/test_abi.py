"""The C-ABI library loads on the host, exports every declared symbol, and its
host-side logic (argument validation, size queries) behaves as documented.
No GPU is needed: every call here returns before any device work."""

import ctypes
import os
import re

import pytest

import block_scaled_fp4_moe_amd as fm
from oracle import permute as OP

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "fp4moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = fm.load()
    names = declared_functions()
    assert len(names) == 21, names
    for n in ["moe_route", "moe_permute", "mxfp4_quant_1x32", "nvfp4_qdq", "fp4_grouped_gemm",
              "moe_combine", "mxfp4_to_fp8_channel", "mxfp4_quant_1x32_chunked",
              "moe_route_permute", "mxfp4_linear"]:
        assert n in names
    for n in names:
        assert getattr(lib, n) is not None


def test_permute_size_queries_match_oracle_bound():
    lib = fm.load()
    for T, topk, E, ns, bm in [(1, 8, 384, 1, 16), (64, 8, 384, 1, 16), (8192, 8, 384, 1, 256),
                               (16, 2, 8, 0, 16), (0, 8, 384, 1, 16), (5, 1, 8, 0, 4)]:
        assert lib.moe_permute_max_tiles(T, topk, E, ns, bm) == OP.max_tiles(T, topk, E, ns, bm)
    assert lib.moe_permute_workspace(64, 8, 384, 1, 16) == 0          # single-launch path
    assert lib.moe_permute_workspace(8192, 8, 384, 1, 256) == 72 * 385 * 4


def _status(call):
    lib = fm.load()
    st = call(lib)
    return st, lib.fp4moe_last_error().decode()


@pytest.mark.parametrize("bad", [
    dict(E=0), dict(E=2000), dict(n_group=5), dict(topk_group=9), dict(topk=0), dict(topk=33),
    dict(n_group=384, topk_group=1)])
def test_route_rejects_bad_arguments(bad):
    a = dict(T=4, E=384, n_group=8, topk_group=4, topk=8)
    a.update(bad)
    st, msg = _status(lambda lib: lib.moe_route(None, None, a["T"], a["E"], a["n_group"],
                                                 a["topk_group"], a["topk"], 1, 1.0, None, None,
                                                 None))
    assert st == 1 and "moe_route" in msg


def test_route_permute_rejects_large_batches():
    def run(T, topk=8, ns=1):
        return _status(lambda lib: lib.moe_route_permute(None, None, T, 384, 8, 4, topk, 1, 1.0, ns,
                                                         16, None, None, None, None, None, None,
                                                         None, None, None))
    st, msg = run(114)                          # 1026 pairs
    assert st == 1 and "1024" in msg
    st, msg = run(4, topk=40)
    assert st == 1 and "topk" in msg
    st, msg = run(4, ns=9)
    assert st == 1 and "n_shared" in msg


def test_quant_and_convert_reject_bad_K():
    st, msg = _status(lambda lib: lib.mxfp4_quant_1x32(None, 4, 48, 48, None, None, None, None,
                                                        None))
    assert st == 1 and "K" in msg
    st, msg = _status(lambda lib: lib.mxfp4_quant_1x32_chunked(None, 4, 96, 96, None, 1, 4, None,
                                                                None, None, None))
    assert st == 1 and "K" in msg               # the chunked layout needs K % 128 == 0
    st, msg = _status(lambda lib: lib.mxfp4_quant_1x32_chunked(None, 4, 128, 128, None, 1, 3, None,
                                                                None, None, None))
    assert st == 1 and "out_rows" in msg        # without a map every input row needs a slot
    st, msg = _status(lambda lib: lib.nvfp4_qdq(None, 4, 24, None, None, None, None, None, None,
                                                 None, None, None, 0, None))
    assert st == 1
    st, msg = _status(lambda lib: lib.nvfp4_qdq(None, 4, 32, None, None, None, None, None, None,
                                                 None, None, None, 0, None))
    assert st == 1 and "null" in msg            # neither y nor y_f16
    st, msg = _status(lambda lib: lib.mxfp4_to_fp8_channel(None, None, 4, 40, None, None, None,
                                                            None, None))
    assert st == 1
    st, msg = _status(lambda lib: lib.mxfp4_to_fp8_channel(None, None, 4, 32800, None, None, None,
                                                            None, None))
    assert st == 1                              # rows up to 32768 values
    st, msg = _status(lambda lib: lib.moe_combine(None, None, None, 2, 8, 1, 7164, None, None,
                                                   None))
    assert st == 1


def test_gemm_rejects_unsupported_combinations():
    def run(**kw):
        a = dict(stage=1, wfmt=0, afmt=0, n_experts=4, N=256, K=256, max_rows=8, max_tiles=4,
                 block_m=16, gather_div=1, lda=256, ldo=128, w_layout=0)
        a.update(kw)
        args = fm.GemmArgs(a["stage"], a["wfmt"], a["afmt"], a["n_experts"], a["N"], a["K"],
                           a["max_rows"], a["max_tiles"], a["block_m"], a["gather_div"],
                           None, None, None, None, None, None, a["lda"], None, None, None, None,
                           None, a["ldo"], a.get("out_f32"), a.get("w_layout", 0),
                           a.get("a_layout", 0), a.get("a_rows", 0), a.get("out_q"),
                           a.get("out_q_scale"), a.get("out_q_rows", 0), a.get("a_f16_scale"),
                           a.get("a_row_scale"), a.get("work_queue"))
        return _status(lambda lib: lib.fp4_grouped_gemm(ctypes.byref(args), None))
    assert run(stage=3)[0] == 1
    assert run(wfmt=1, afmt=1)[0] == 1          # NVFP4 weights need bf16 activations
    assert run(wfmt=3)[0] == 1
    assert run(afmt=2)[0] == 1
    assert run(K=96)[0] == 1
    assert run(block_m=128)[0] == 1             # bf16 path tiles are 16/32/64 rows
    assert run(wfmt=2, afmt=1, block_m=128)[0] == 1
    assert run(afmt=1, block_m=16)[0] == 1
    assert run(N=96)[0] == 1
    assert run(w_layout=2)[0] == 1
    assert run(a_layout=2)[0] == 1
    # chunked activations: MXFP4 x MXFP4, fragment weights, block_m 128 / 192 / 256 only
    assert run(afmt=1, block_m=128, w_layout=1, a_layout=1, a_rows=8, max_tiles=0)[0] == 0
    assert run(afmt=1, block_m=64, w_layout=1, a_layout=1, a_rows=8)[0] == 1
    assert run(afmt=1, block_m=128, w_layout=0, a_layout=1, a_rows=8)[0] == 1
    assert run(afmt=0, block_m=16, w_layout=1, a_layout=1, a_rows=8)[0] == 1
    assert run(afmt=1, block_m=128, w_layout=1, a_layout=1, a_rows=4)[0] == 1   # < max_rows
    # block_m 192: MXFP4 x MXFP4 with fragment weights, output width a multiple
    # of 256 (stage 1) / 512 (stage 2)
    wide = dict(afmt=1, block_m=192, w_layout=1, N=512, ldo=512)
    assert run(**wide, max_tiles=0)[0] == 0
    assert run(**{**wide, "w_layout": 0})[0] == 1
    assert run(**{**wide, "N": 256})[0] == 1
    assert run(**{**wide, "N": 256}, stage=2, max_tiles=0)[0] == 1
    assert run(**wide, stage=2, max_tiles=0)[0] == 0
    assert run(**wide, a_layout=1, a_rows=8, max_tiles=0)[0] == 0
    assert run(**wide, a_layout=1, a_rows=0, max_rows=0, max_tiles=0)[0] == 0   # empty batch
    assert run(**wide, a_layout=1, a_rows=0, max_tiles=0)[0] == 1               # rows but no slab
    assert run(**{**wide, "block_m": 160})[0] == 1
    assert run(**{**wide, "ldo": 516}, max_tiles=0)[0] == 1     # 16-byte row stores
    # FP8 weights x MXFP4 activations at block_m 192 (192 x 256 tiles)
    wide8 = dict(wfmt=2, afmt=1, block_m=192, w_layout=1, N=256, ldo=256)
    assert run(**wide8, max_tiles=0)[0] == 0
    assert run(**wide8, stage=2, max_tiles=0)[0] == 0
    assert run(**wide8, a_layout=1, a_rows=8, max_tiles=0)[0] == 0
    assert run(**{**wide8, "w_layout": 0}, max_tiles=0)[0] == 1
    assert run(**{**wide8, "N": 320}, max_tiles=0)[0] == 1       # output width 160
    assert run(**{**wide8, "N": 128}, stage=2, max_tiles=0)[0] == 1
    assert run(**{**wide8, "afmt": 0}, max_tiles=0)[0] == 1      # bf16 activations: 16/32/64
    # stage-1 output quantized in the epilogue: block_m 192, MXFP4 activations,
    # both buffers, no fp32 copy, enough rows (pointers are never touched here)
    q = dict(out_q=64, out_q_scale=128, out_q_rows=8, max_tiles=0)
    assert run(**wide, **q)[0] == 0
    assert run(**wide8, **q)[0] == 0
    assert run(**wide, **{**q, "out_q_scale": None})[0] == 1
    assert run(**wide, **q, stage=2)[0] == 1
    assert run(**{**wide, "block_m": 256, "ldo": 256}, **q)[0] == 1
    assert run(**wide, **{**q, "out_q_rows": 4})[0] == 1       # < max_rows
    # W8A8: FP8 weights x FP8 activations, block_m 128, fragment weights,
    # chunk-major activations, a row-scale pointer, output width a multiple of
    # 128 (stage 1) / 256 (stage 2), no quantized stage-1 output
    w8a8 = dict(wfmt=2, afmt=3, block_m=128, w_layout=1, a_layout=1, a_rows=8, N=256, ldo=256)
    assert run(**w8a8, max_tiles=0)[0] == 0
    assert run(**w8a8, stage=2, max_tiles=0)[0] == 0
    assert run(**{**w8a8, "wfmt": 0}, max_tiles=0)[0] == 1      # MXFP4 weights
    assert run(**{**w8a8, "block_m": 192}, max_tiles=0)[0] == 1
    assert run(**{**w8a8, "w_layout": 0}, max_tiles=0)[0] == 1
    assert run(**{**w8a8, "a_layout": 0}, max_tiles=0)[0] == 1
    assert run(**{**w8a8, "N": 320}, max_tiles=0)[0] == 1       # output width 160
    assert run(**w8a8, **q)[0] == 1
    assert run(**w8a8)[0] == 1                                   # null pointers with work
    assert run(**wide, **q, out_f32=256)[0] == 1
    # f16 activations (the NVFP4 operand form): NVFP4 fragment weights, block_m 64
    f16 = dict(wfmt=1, afmt=2, block_m=64, w_layout=1, N=512, ldo=256, max_tiles=0)
    assert run(**f16)[0] == 0
    assert run(**{**f16, "ldo": 512}, stage=2)[0] == 0
    assert run(**{**f16, "wfmt": 0})[0] == 1
    assert run(**{**f16, "block_m": 16})[0] == 1
    assert run(**{**f16, "w_layout": 0})[0] == 1
    assert run(**{**f16, "N": 192, "ldo": 96})[0] == 1           # output width 96
    # block_m 128: the 128-row tiles, K a multiple of 512
    assert run(**{**f16, "block_m": 128, "K": 512, "lda": 512})[0] == 0
    assert run(**{**f16, "block_m": 128, "K": 512, "lda": 512, "ldo": 512}, stage=2)[0] == 0
    st, msg = run(**{**f16, "block_m": 128, "K": 384, "lda": 384})
    assert st == 1 and "512" in msg
    assert run(**{**f16, "block_m": 192, "K": 512, "lda": 512})[0] == 1
    # the work queue: any 4-byte aligned device pointer (never touched here)
    assert run(**{**f16, "block_m": 128, "K": 512, "lda": 512}, work_queue=256)[0] == 0
    st, msg = run(**{**f16, "block_m": 128, "K": 512, "lda": 512}, work_queue=258)
    assert st == 1 and "work_queue" in msg
    assert run(afmt=3)[0] == 1
    assert run(max_tiles=0)[0] == 0             # nothing to do: OK without touching pointers


def test_linear_rejects_bad_arguments():
    def run(M=8, K=256, layout=0, stride=256, N=512, ldo=512):
        return _status(lambda lib: lib.mxfp4_linear(None, None, M, K, layout, stride, None, None,
                                                    N, None, ldo, None, None))
    assert run(M=0)[0] == 0                     # nothing to do
    assert run()[0] == 1                        # null pointers
    for bad in (dict(K=96), dict(N=256), dict(layout=2), dict(ldo=516), dict(ldo=256),
                dict(stride=128), dict(layout=1, stride=4), dict(M=-1)):
        st, msg = run(**bad)
        assert st == 1 and "mxfp4_linear" in msg, bad
    assert run(M=0, layout=1, stride=0)[0] == 0


def test_combine_takes_more_than_65535_tokens():
    """The token count has no cap below the int range: T = 65536 passes the
    argument checks (on a host without a gfx950 device the call then stops at
    the device check, before any launch)."""
    fake = ctypes.c_void_p(4096)
    st, msg = _status(lambda lib: lib.moe_combine(fake, fake, fake, 65536, 8, 1, 64, fake, None,
                                                   None))
    assert st != 1, msg


def test_too_small_workspace_is_reported():
    """The multi-launch permutation and the dynamic NVFP4 scale need caller
    workspace; too little returns FP4MOE_ERR_WORKSPACE (3) before any launch
    (the pointers below are never dereferenced)."""
    fake = ctypes.c_void_p(4096)
    need = fm.load().moe_permute_workspace(200, 8, 384, 1, 16)
    assert need > 0
    for ws, nbytes in ((None, 0), (fake, need - 4)):
        st, msg = _status(lambda lib: lib.moe_permute(fake, 200, 8, 384, 1, 16, ws, nbytes, fake,
                                                      fake, fake, fake, fake, fake, None))
        assert st == 3 and "workspace" in msg
    st, msg = _status(lambda lib: lib.nvfp4_qdq(fake, 4, 32, None, None, fake, None, None, None,
                                                 None, None, None, 0, None))
    assert st == 3 and "nvfp4_qdq" in msg


def test_preshuffle_rejects_bad_shapes():
    st, msg = _status(lambda lib: lib.fp4_weight_preshuffle(0, 2, 24, 256, None, None, None,
                                                             None, None))
    assert st == 1 and "N" in msg
    st, msg = _status(lambda lib: lib.fp4_weight_preshuffle(0, 2, 32, 192, None, None, None,
                                                             None, None))
    assert st == 1
    assert _status(lambda lib: lib.fp4_weight_preshuffle(0, 0, 32, 256, None, None, None, None,
                                                          None))[0] == 0


def test_permute_noalloc_rejects_batches_beyond_its_buffer():
    """The library-owned histogram buffer is 4 MiB: a batch needing more is
    refused before any device work (the pointers are never dereferenced)."""
    lib = fm.load()
    cap = lib.moe_permute_noalloc_max_workspace()
    assert cap == 4 << 20
    T, topk, E, ns, bm = 40000, 8, 4000, 0, 64
    assert lib.moe_permute_workspace(T, topk, E, ns, bm) > cap
    p = ctypes.c_void_p(256)
    st, msg = _status(lambda lib: lib.moe_permute_noalloc(p, T, topk, E, ns, bm, p, p, p, p, p, p,
                                                          None))
    assert st == 3 and "moe_permute_noalloc" in msg and "4194304" in msg


def _decode_args(**kw):
    a = fm.DecodeArgs(T=1, H=7168, I=2048, E=384, n_shared=1, n_group=8, topk_group=4, topk=8,
                      renormalize=1, max_tiles=9, routed_scale=1.0)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("bad", [dict(T=17), dict(T=-1), dict(topk=17), dict(n_shared=9),
                                 dict(H=7000), dict(I=2000), dict(E=1100), dict(n_group=5),
                                 dict(max_tiles=8), dict(workspace_bytes=16)])
def test_decode_fused_rejects_bad_arguments(bad):
    """Argument and workspace checks of the single-launch decode, before any
    device work (the pointers are never dereferenced): FP4MOE_ERR_INVALID_ARG,
    or FP4MOE_ERR_WORKSPACE for a workspace below moe_decode_fused_workspace."""
    lib = fm.load()
    ws = lib.moe_decode_fused_workspace(7168)
    assert ws == (4 + 112) * 4
    a = _decode_args(**{"workspace_bytes": ws, **bad})
    st, msg = _status(lambda lib: lib.moe_decode_fused(ctypes.byref(a), None))
    want = 3 if "workspace_bytes" in bad else 1
    assert st == want and "moe_decode_fused" in msg, (bad, st, msg)
    # T = 0 with valid sizes is accepted and does nothing
    a = _decode_args(T=0, max_tiles=0, workspace_bytes=ws)
    assert _status(lambda lib: lib.moe_decode_fused(ctypes.byref(a), None))[0] == 0


def test_fp8_quant_rejects_bad_arguments():
    """Shape and layout checks of fp8_quant_per_token before any device work."""
    fake = ctypes.c_void_p(4096)
    for M, K, ldx, out_rows in [(4, 96, 96, 4), (4, 8320, 8320, 4), (4, 256, 200, 4),
                                (4, 256, 256, 3), (-1, 256, 256, 4)]:
        st, msg = _status(lambda lib: lib.fp8_quant_per_token(fake, M, K, ldx, None, out_rows,
                                                              fake, fake, None))
        assert st == 1 and "fp8_quant_per_token" in msg, (M, K, ldx, out_rows, msg)
    assert _status(lambda lib: lib.fp8_quant_per_token(None, 0, 256, 256, None, 0, None, None,
                                                       None))[0] == 0


def test_layer_buffer_cache_is_bounded():
    """The layer keeps its intermediate buffers for the most recently used
    batch sizes only (host-side sizing; the buffers live on the CPU here)."""
    from block_scaled_fp4_moe_amd import layer as L
    cfg = fm.LayerConfig(H=256, I=128, E=8, n_shared=1, n_group=1, topk_group=1, topk=2,
                         afmt="bf16", wfmt="mx", block_m=16, fragment_layout=False)
    lay = fm.MoELayer(cfg, {}, device="cpu")
    sizes = list(range(1, L.MAX_CACHED_BATCH_SIZES + 5))
    for T in sizes:
        b = lay._buffers(T)
        assert b["h"].shape == (T * 3, 128) and b["out"].shape == (T, 256)
    assert list(lay._bufs) == sizes[-L.MAX_CACHED_BATCH_SIZES:]
    again = lay._buffers(sizes[-L.MAX_CACHED_BATCH_SIZES])     # a hit moves to the back
    assert again is lay._bufs[sizes[-L.MAX_CACHED_BATCH_SIZES]]
    assert list(lay._bufs)[-1] == sizes[-L.MAX_CACHED_BATCH_SIZES]
