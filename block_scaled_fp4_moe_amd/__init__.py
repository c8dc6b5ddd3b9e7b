"""Python binding of libfp4moe (the C ABI declared in include/fp4moe.h).

Argument marshalling only: every step runs in the HIP kernels of the
library.  PyTorch provides device memory and the current HIP stream; the
functions take and return torch tensors.  There is no fallback: if the
library is not built or the device is not gfx950, calls raise.

Entry points (same names as the C ABI): moe_route, moe_permute,
mxfp4_quant_1x32, nvfp4_qdq, fp8_quant_per_token, fp4_grouped_gemm,
moe_combine, mxfp4_to_fp8_channel, moe_decode_fused, and the helpers the
header declares.  `MoELayer` (layer.py) chains them into the layer.
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp4moe.so")

W_MXFP4, W_NVFP4, W_FP8 = 0, 1, 2
A_BF16, A_MXFP4, A_F16, A_FP8 = 0, 1, 2, 3
LAYOUT_ROWMAJOR, LAYOUT_FRAGMENT = 0, 1
A_LAYOUT_ROWMAJOR, A_LAYOUT_CHUNKED = 0, 1
WFMT = {"mx": W_MXFP4, "nvfp4": W_NVFP4, "fp8": W_FP8}

_lib = None


class FP4MoEError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"fp4moe status {status}: {msg}")
        self.status = status


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int), ("H", ctypes.c_int), ("I", ctypes.c_int), ("E", ctypes.c_int),
        ("n_shared", ctypes.c_int), ("n_group", ctypes.c_int), ("topk_group", ctypes.c_int),
        ("topk", ctypes.c_int), ("renormalize", ctypes.c_int), ("max_tiles", ctypes.c_int),
        ("routed_scale", ctypes.c_float),
        ("x", ctypes.c_void_p), ("logits", ctypes.c_void_p), ("bias", ctypes.c_void_p),
        ("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p), ("w2", ctypes.c_void_p),
        ("w2_scale", ctypes.c_void_p),
        ("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
        ("expert_offsets", ctypes.c_void_p), ("sorted_pairs", ctypes.c_void_p),
        ("pair_pos", ctypes.c_void_p), ("tiles", ctypes.c_void_p), ("n_tiles", ctypes.c_void_p),
        ("n_dropped", ctypes.c_void_p), ("h", ctypes.c_void_p), ("y", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class GemmArgs(ctypes.Structure):
    _fields_ = [
        ("stage", ctypes.c_int), ("wfmt", ctypes.c_int), ("afmt", ctypes.c_int),
        ("n_experts", ctypes.c_int), ("N", ctypes.c_int), ("K", ctypes.c_int),
        ("max_rows", ctypes.c_int), ("max_tiles", ctypes.c_int), ("block_m", ctypes.c_int),
        ("gather_div", ctypes.c_int),
        ("w", ctypes.c_void_p), ("w_scale", ctypes.c_void_p),
        ("w_tensor_scale", ctypes.c_void_p), ("w_channel_scale", ctypes.c_void_p),
        ("a", ctypes.c_void_p), ("a_scale", ctypes.c_void_p), ("lda", ctypes.c_int64),
        ("a_row_gather", ctypes.c_void_p), ("expert_offsets", ctypes.c_void_p),
        ("tiles", ctypes.c_void_p), ("n_tiles", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("ldo", ctypes.c_int64), ("out_f32", ctypes.c_void_p),
        ("w_layout", ctypes.c_int), ("a_layout", ctypes.c_int), ("a_rows", ctypes.c_int),
        ("out_q", ctypes.c_void_p), ("out_q_scale", ctypes.c_void_p), ("out_q_rows", ctypes.c_int),
        ("a_f16_scale", ctypes.c_void_p), ("a_row_scale", ctypes.c_void_p),
        ("work_queue", ctypes.c_void_p),
    ]


def load():
    """Load libfp4moe.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run python -m block_scaled_fp4_moe_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "fp4moe_last_error": ([], ctypes.c_char_p),
        "fp4moe_init": ([], I),
        "moe_route": ([P, P, I, I, I, I, I, I, F, P, P, P], I),
        "moe_permute_max_tiles": ([I, I, I, I, I], I),
        "moe_permute_workspace": ([I, I, I, I, I], S),
        "moe_permute": ([P, I, I, I, I, I, P, S, P, P, P, P, P, P, P], I),
        "moe_permute_noalloc_max_workspace": ([], S),
        "moe_permute_noalloc": ([P, I, I, I, I, I, P, P, P, P, P, P, P], I),
        "moe_route_permute": ([P, P, I, I, I, I, I, I, F, I, I, P, P, P, P, P, P, P, P, P], I),
        "mxfp4_quant_1x32": ([P, I, I, I64, P, P, P, P, P], I),
        "mxfp4_quant_1x32_chunked": ([P, I, I, I64, P, I, I, P, P, P, P], I),
        "fp8_quant_per_token": ([P, I, I, I64, P, I, P, P, P], I),
        "nvfp4_qdq_workspace": ([], S),
        "nvfp4_qdq": ([P, I, I, P, P, P, P, P, P, P, P, P, S, P], I),
        "fp4_grouped_gemm": ([ctypes.POINTER(GemmArgs), P], I),
        "mxfp4_linear": ([P, P, I, I, I, I64, P, P, I, P, I64, P, P], I),
        "moe_combine": ([P, P, P, I, I, I, I, P, P, P], I),
        "fp4_weight_preshuffle": ([I, I, I, I, P, P, P, P, P], I),
        "mxfp4_to_fp8_channel": ([P, P, I64, I, P, P, P, P, P], I),
        "moe_decode_fused_workspace": ([I], S),
        "moe_decode_fused": ([ctypes.POINTER(DecodeArgs), P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        raise FP4MoEError(status, load().fp4moe_last_error().decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t):
    return t.device


def _u16(x):
    """bf16 / f16 tensor (or its int16/uint16 bit view) -> int16 view for pointer passing."""
    if x.dtype in (torch.bfloat16, torch.float16):
        return x.view(torch.int16)
    assert x.dtype in (torch.int16, torch.uint16), x.dtype
    return x


# ---------------------------------------------------------------- entry points

def moe_route(logits, bias, n_group, topk_group, topk, renormalize=True, routed_scale=1.0,
              topk_ids=None, topk_w=None, stream=None):
    lib = load()
    T, E = logits.shape
    assert logits.dtype == torch.float32 and logits.is_contiguous()
    if topk_ids is None:
        topk_ids = torch.empty((T, topk), dtype=torch.int32, device=_dev(logits))
    if topk_w is None:
        topk_w = torch.empty((T, topk), dtype=torch.float32, device=_dev(logits))
    _check(lib.moe_route(_p(logits), _p(bias), T, E, n_group, topk_group, topk,
                         int(bool(renormalize)), float(routed_scale), _p(topk_ids), _p(topk_w),
                         _stream(stream)))
    return topk_ids, topk_w


def moe_permute_max_tiles(T, topk, E, n_shared, block_m):
    return load().moe_permute_max_tiles(T, topk, E, n_shared, block_m)


def moe_permute(topk_ids, E, n_shared, block_m, workspace=None, out=None, stream=None):
    """Returns a dict of device tensors: expert_offsets, sorted_pairs, pair_pos,
    tiles, n_tiles, n_dropped (and max_tiles as a Python int)."""
    lib = load()
    T, topk = topk_ids.shape
    k = topk + n_shared
    dev = _dev(topk_ids)
    mt = lib.moe_permute_max_tiles(T, topk, E, n_shared, block_m)
    if out is None:
        out = dict(
            expert_offsets=torch.empty(E + n_shared + 1, dtype=torch.int32, device=dev),
            sorted_pairs=torch.empty(T * k, dtype=torch.int32, device=dev),
            pair_pos=torch.empty(T * k, dtype=torch.int32, device=dev),
            tiles=torch.empty((max(mt, 1), 2), dtype=torch.int32, device=dev),
            n_tiles=torch.empty(1, dtype=torch.int32, device=dev),
            n_dropped=torch.empty(1, dtype=torch.int32, device=dev))
    out["max_tiles"] = mt
    need = lib.moe_permute_workspace(T, topk, E, n_shared, block_m)
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(lib.moe_permute(_p(topk_ids.contiguous()), T, topk, E, n_shared, block_m,
                           _p(workspace) if need else None, need,
                           _p(out["expert_offsets"]), _p(out["sorted_pairs"]), _p(out["pair_pos"]),
                           _p(out["tiles"]), _p(out["n_tiles"]), _p(out["n_dropped"]),
                           _stream(stream)))
    return out


def moe_permute_noalloc(topk_ids, E, n_shared, block_m, out, stream=None):
    """moe_permute without a workspace argument: the library's own per-device
    buffer holds the chunk histograms.  `out` holds the caller's output
    tensors (the dict moe_permute returns); nothing is allocated here."""
    lib = load()
    T, topk = topk_ids.shape
    assert topk_ids.is_contiguous()
    _check(lib.moe_permute_noalloc(_p(topk_ids), T, topk, E, n_shared, block_m,
                                   _p(out["expert_offsets"]), _p(out["sorted_pairs"]),
                                   _p(out["pair_pos"]), _p(out["tiles"]), _p(out["n_tiles"]),
                                   _p(out["n_dropped"]), _stream(stream)))
    return out


def moe_route_permute(logits, bias, n_group, topk_group, topk, n_shared, block_m,
                      renormalize=True, routed_scale=1.0, topk_ids=None, topk_w=None, out=None,
                      stream=None):
    """moe_route then moe_permute in one launch (T * (topk + n_shared) <= 1024).
    Returns (topk_ids, topk_w, perm) with perm as moe_permute returns it."""
    lib = load()
    T, E = logits.shape
    assert logits.dtype == torch.float32 and logits.is_contiguous()
    dev = _dev(logits)
    k = topk + n_shared
    if topk_ids is None:
        topk_ids = torch.empty((T, topk), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, topk), dtype=torch.float32, device=dev)
    mt = lib.moe_permute_max_tiles(T, topk, E, n_shared, block_m)
    if out is None:
        out = dict(
            expert_offsets=torch.empty(E + n_shared + 1, dtype=torch.int32, device=dev),
            sorted_pairs=torch.empty(T * k, dtype=torch.int32, device=dev),
            pair_pos=torch.empty(T * k, dtype=torch.int32, device=dev),
            tiles=torch.empty((max(mt, 1), 2), dtype=torch.int32, device=dev),
            n_tiles=torch.empty(1, dtype=torch.int32, device=dev),
            n_dropped=torch.empty(1, dtype=torch.int32, device=dev))
    out["max_tiles"] = mt
    _check(lib.moe_route_permute(_p(logits), _p(bias), T, E, n_group, topk_group, topk,
                                 int(bool(renormalize)), float(routed_scale), n_shared, block_m,
                                 _p(topk_ids), _p(topk_w), _p(out["expert_offsets"]),
                                 _p(out["sorted_pairs"]), _p(out["pair_pos"]), _p(out["tiles"]),
                                 _p(out["n_tiles"]), _p(out["n_dropped"]), _stream(stream)))
    return topk_ids, topk_w, out


def mxfp4_quant_1x32(x, row_gather=None, row_count=None, codes=None, scales=None, M=None,
                     stream=None):
    """x bf16 [rows, K] (row stride taken from x) -> (codes uint8 [M, K/2], scales uint8 [M, K/32])."""
    lib = load()
    xs = _u16(x)
    K = xs.shape[1]
    if M is None:
        M = row_gather.shape[0] if row_gather is not None else xs.shape[0]
    assert xs.stride(1) == 1
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=_dev(x))
    if scales is None:
        scales = torch.empty((M, K // 32), dtype=torch.uint8, device=_dev(x))
    _check(lib.mxfp4_quant_1x32(_p(xs), M, K, xs.stride(0), _p(row_gather), _p(row_count),
                                _p(codes), _p(scales), _stream(stream)))
    return codes, scales


def mxfp4_quant_1x32_chunked(x, row_map=None, map_k=1, out_rows=None, row_count=None,
                             codes=None, scales=None, stream=None):
    """x bf16 [M, K] -> chunk-major (codes uint8 [K/128, out_rows, 64], scales [K/128, out_rows, 4]).

    Input row r goes to output rows row_map[r*map_k + j] (j < map_k), or to row r."""
    lib = load()
    xs = _u16(x)
    M, K = xs.shape
    if out_rows is None:
        out_rows = codes.shape[1] if codes is not None else (M * map_k if row_map is not None else M)
    assert xs.stride(1) == 1
    if codes is None:
        codes = torch.empty((K // 128, out_rows, 64), dtype=torch.uint8, device=_dev(x))
    if scales is None:
        scales = torch.empty((K // 128, out_rows, 4), dtype=torch.uint8, device=_dev(x))
    _check(lib.mxfp4_quant_1x32_chunked(_p(xs), M, K, xs.stride(0), _p(row_map), map_k, out_rows,
                                        _p(row_count), _p(codes), _p(scales), _stream(stream)))
    return codes, scales


def nvfp4_qdq(x, tensor_scale=None, row_count=None, y=None, codes=None, scales=None,
              tensor_scale_out=None, y_f16=None, y_f16_scale=None, no_y=False, workspace=None,
              stream=None):
    """x bf16 [M, K] -> y bf16 [M, K] (and optional codes, scales, tensor scale, and
    the f16 operand form y_f16 [M, K] float16 with its factor y_f16_scale [1]).
    With no_y=True (y_f16 given) y is not written and None is returned."""
    lib = load()
    xs = _u16(x).contiguous()
    M, K = xs.shape
    if y is None and not no_y:
        y = torch.empty((M, K), dtype=torch.bfloat16, device=_dev(x))
    if workspace is None and tensor_scale is None:
        workspace = torch.empty(lib.nvfp4_qdq_workspace(), dtype=torch.uint8, device=_dev(x))
    _check(lib.nvfp4_qdq(_p(xs), M, K, _p(row_count), _p(tensor_scale),
                         None if y is None else _p(_u16(y)), _p(codes), _p(scales),
                         _p(tensor_scale_out), None if y_f16 is None else _p(_u16(y_f16)),
                         _p(y_f16_scale), _p(workspace),
                         0 if workspace is None else workspace.numel(), _stream(stream)))
    return y


def fp4_grouped_gemm(stage, wfmt, afmt, w, w_scale, a, perm, block_m, *, a_scale=None,
                     w_tensor_scale=None, w_channel_scale=None, a_row_gather=None,
                     gather_div=1, out=None, out_f32=None, max_rows=None, w_layout=0,
                     a_layout=0, out_q=None, out_q_scale=None, no_out=False, a_f16_scale=None,
                     a_row_scale=None, work_queue=None, stream=None):
    """One GEMM stage over the expert segments described by `perm` (moe_permute output).

    w: weight codes [E, N, K/2] (FP8: [E, N, K]); a: bf16 [rows, K] or MXFP4
    codes [rows, K/2] with a_scale [rows, K/32] (a_layout 0), or chunk-major
    MXFP4 codes [K/128, rows, 64] with a_scale [K/128, rows, 4] (a_layout 1).
    afmt A_F16: a is the f16 operand form of nvfp4_qdq (viewed as int16 / float16)
    and a_f16_scale its float32 [1] power-of-two factor.
    afmt A_FP8 (FP8 weights, block_m 128): a is fp8_quant_per_token's chunk-major
    E4M3 codes [K/128, rows, 128] and a_row_scale its float32 [rows] scales.
    work_queue (A_F16 at block_m 128): an int32 [16] tensor, zero-filled once;
    the workgroups then take their items from it as they free up.
    out_q / out_q_scale (stage 1, block_m 192): chunk-major MXFP4 copies of the
    output [N_out/128, rows, 64] / [N_out/128, rows, 4]; with no_out=True the
    bf16 output is not written (returns None).
    Returns out bf16 [max_rows, N_out]."""
    lib = load()
    E, N = w.shape[0], w.shape[1]
    K = w.shape[2] if wfmt == W_FP8 else w.shape[2] * 2
    n_out = N // 2 if stage == 1 else N
    if max_rows is None:
        max_rows = perm["sorted_pairs"].shape[0]
    a_rows = 0
    if afmt in (A_BF16, A_F16):
        a_ = _u16(a)
        lda = a_.stride(0)
    elif a_layout == A_LAYOUT_CHUNKED:
        a_ = a
        a_rows = a.shape[1]
        lda = K
    else:
        a_ = a
        lda = a.stride(0) * 2
    if out is None and not no_out:
        out = torch.empty((max_rows, n_out), dtype=torch.bfloat16, device=_dev(a))
    args = GemmArgs(stage, wfmt, afmt, E, N, K, max_rows, perm["max_tiles"], block_m, gather_div,
                    w.data_ptr(), None if w_scale is None else w_scale.data_ptr(),
                    None if w_tensor_scale is None else w_tensor_scale.data_ptr(),
                    None if w_channel_scale is None else w_channel_scale.data_ptr(),
                    a_.data_ptr(), None if a_scale is None else a_scale.data_ptr(), lda,
                    None if a_row_gather is None else a_row_gather.data_ptr(),
                    perm["expert_offsets"].data_ptr(), perm["tiles"].data_ptr(),
                    perm["n_tiles"].data_ptr(), None if out is None else out.data_ptr(),
                    n_out if out is None else out.stride(0),
                    None if out_f32 is None else out_f32.data_ptr(), w_layout, a_layout, a_rows,
                    None if out_q is None else out_q.data_ptr(),
                    None if out_q_scale is None else out_q_scale.data_ptr(),
                    0 if out_q is None else out_q.shape[1],
                    None if a_f16_scale is None else a_f16_scale.data_ptr(),
                    None if a_row_scale is None else a_row_scale.data_ptr(),
                    None if work_queue is None else work_queue.data_ptr())
    _check(lib.fp4_grouped_gemm(ctypes.byref(args), _stream(stream)))
    return out


def fp8_quant_per_token(x, row_count=None, out_rows=None, codes=None, scales=None, stream=None):
    """Dynamic per-token FP8 of bf16 rows x [M, K]: codes chunk-major
    [K/128, out_rows, 128] (uint8 E4M3) and scales float32 [out_rows]."""
    lib = load()
    M, K = x.shape
    out_rows = M if out_rows is None else out_rows
    if codes is None:
        codes = torch.empty((K // 128, out_rows, 128), dtype=torch.uint8, device=_dev(x))
    if scales is None:
        scales = torch.empty(out_rows, dtype=torch.float32, device=_dev(x))
    x_ = _u16(x)
    _check(lib.fp8_quant_per_token(_p(x_), M, K, x_.stride(0), _p(row_count), out_rows,
                                   _p(codes), _p(scales), _stream(stream)))
    return codes, scales


def mxfp4_linear(a, a_scale, w, w_scale, a_layout=0, M=None, out=None, out_f32=None,
                 stream=None):
    """Dense out = bf16(A . W^T): a / a_scale MXFP4 activations (row-major codes
    [M, K/2] + scales [M, K/32], or chunk-major [K/128, rows, 64] / [K/128, rows, 4]
    with a_layout 1 and M <= rows), w / w_scale one fragment-major MXFP4 matrix
    [N, K/2] / [N, K/32] (fp4_weight_preshuffle of a [1, N, K/2] tensor).
    Returns out bf16 [M, N]."""
    lib = load()
    N, K = w.shape[-2], w.shape[-1] * 2
    if a_layout == A_LAYOUT_CHUNKED:
        rows = a.shape[1]
        M = rows if M is None else M
        stride = rows
    else:
        M = a.shape[0] if M is None else M
        stride = a.stride(0) * 2
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=_dev(a))
    _check(lib.mxfp4_linear(_p(a), _p(a_scale), M, K, a_layout, stride, _p(w), _p(w_scale), N,
                            _p(_u16(out)), out.stride(0), _p(out_f32), _stream(stream)))
    return out


def fp4_weight_preshuffle(wfmt, codes, scales=None, codes_out=None, scales_out=None,
                          stream=None):
    """Expert weights [E, N, K/2] (FP8 [E, N, K]) + scales -> fragment-major copies."""
    lib = load()
    E, N = codes.shape[0], codes.shape[1]
    K = codes.shape[2] if wfmt == W_FP8 else codes.shape[2] * 2
    if codes_out is None:
        codes_out = torch.empty_like(codes)
    if scales is not None and scales_out is None and wfmt != W_FP8:
        scales_out = torch.empty_like(scales)
    _check(lib.fp4_weight_preshuffle(wfmt, E, N, K, _p(codes), _p(scales if wfmt != W_FP8 else None),
                                     _p(codes_out), _p(scales_out if wfmt != W_FP8 else None),
                                     _stream(stream)))
    return codes_out, (scales_out if wfmt != W_FP8 else scales)


def moe_combine(y, pair_pos, topk_w, topk, n_shared, out=None, out_f32=None, stream=None):
    lib = load()
    T = topk_w.shape[0]
    H = y.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=_dev(y))
    _check(lib.moe_combine(_p(_u16(y)), _p(pair_pos), _p(topk_w), T, topk, n_shared, H,
                           _p(_u16(out)), _p(out_f32), _stream(stream)))
    return out


def mxfp4_to_fp8_channel(codes, scales, fp8=None, channel_scale=None, row_status=None,
                         n_inexact=None, stream=None):
    """codes [rows, K/2], scales [rows, K/32] -> (fp8 [rows, K], scale f32 [rows],
    row_status u8 [rows], n_inexact u32 [1])."""
    lib = load()
    rows = codes.shape[0]
    K = codes.shape[1] * 2
    dev = _dev(codes)
    if fp8 is None:
        fp8 = torch.empty((rows, K), dtype=torch.uint8, device=dev)
    if channel_scale is None:
        channel_scale = torch.empty(rows, dtype=torch.float32, device=dev)
    if row_status is None:
        row_status = torch.empty(rows, dtype=torch.uint8, device=dev)
    if n_inexact is None:
        n_inexact = torch.empty(1, dtype=torch.int32, device=dev)
    _check(lib.mxfp4_to_fp8_channel(_p(codes), _p(scales), rows, K, _p(fp8), _p(channel_scale),
                                    _p(row_status), _p(n_inexact), _stream(stream)))
    return fp8, channel_scale, row_status, n_inexact


def moe_decode_fused(x, logits, bias, w13, w13_scale, w2, w2_scale, *, I, n_shared, n_group,
                     topk_group, topk, workspace, out, renormalize=True, routed_scale=1.0,
                     stream=None):
    """The whole decode layer (T <= 16, bf16 activations, fragment-major MXFP4
    weights) in one launch.  `out` holds the caller's buffers: topk_ids, topk_w,
    perm (the dict moe_permute returns, tiles sized for block_m 16), h, y and
    out.  `workspace`: moe_decode_fused_workspace(H) bytes, zero-filled before
    the first call (uint8 or int32 tensor)."""
    lib = load()
    T, H = x.shape
    E = logits.shape[1]
    perm = out["perm"]
    a = DecodeArgs(T=T, H=H, I=I, E=E, n_shared=n_shared, n_group=n_group,
                   topk_group=topk_group, topk=topk, renormalize=int(bool(renormalize)),
                   max_tiles=perm["tiles"].shape[0], routed_scale=float(routed_scale),
                   x=x.data_ptr(), logits=logits.data_ptr(),
                   bias=bias.data_ptr() if bias is not None else None,
                   w13=w13.data_ptr(), w13_scale=w13_scale.data_ptr(), w2=w2.data_ptr(),
                   w2_scale=w2_scale.data_ptr(),
                   topk_ids=out["topk_ids"].data_ptr(), topk_w=out["topk_w"].data_ptr(),
                   expert_offsets=perm["expert_offsets"].data_ptr(),
                   sorted_pairs=perm["sorted_pairs"].data_ptr(),
                   pair_pos=perm["pair_pos"].data_ptr(), tiles=perm["tiles"].data_ptr(),
                   n_tiles=perm["n_tiles"].data_ptr(), n_dropped=perm["n_dropped"].data_ptr(),
                   h=out["h"].data_ptr(), y=out["y"].data_ptr(), out=out["out"].data_ptr(),
                   workspace=workspace.data_ptr(),
                   workspace_bytes=workspace.numel() * workspace.element_size())
    _check(lib.moe_decode_fused(ctypes.byref(a), _stream(stream)))
    return out



from .layer import MoELayer, LayerConfig  # noqa: E402,F401

