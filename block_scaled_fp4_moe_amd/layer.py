"""The MoE layer as a chain of the C-ABI calls (marshalling and buffer reuse only).

Order ([ATOM] "Stage D: MXFP4 Fused MoE", [NVFP4] "Weight Dequantization and
Activation QDQ"): moe_route -> moe_permute (one launch, moe_route_permute, at
decode sizes) -> activation quantization
(mxfp4_quant_1x32 | nvfp4_qdq | none) -> fp4_grouped_gemm stage 1 (gate/up,
SiLU*up) -> quantization of h (in the stage-1 epilogue for 192-row tiles) ->
fp4_grouped_gemm stage 2 (down) ->
moe_combine.  Decode batches of at most 16 tokens with bf16 activations and
MXFP4 weights take all of it in one launch (moe_decode_fused) instead.
Every step is a kernel of libfp4moe; this module only allocates device
buffers (once per token count) and passes pointers.
"""

from collections import OrderedDict
from dataclasses import dataclass

import torch

from . import (A_BF16, A_F16, A_FP8, A_LAYOUT_CHUNKED, A_LAYOUT_ROWMAJOR, A_MXFP4,
               LAYOUT_FRAGMENT, LAYOUT_ROWMAJOR, WFMT, fp4_grouped_gemm, fp4_weight_preshuffle,
               fp8_quant_per_token, moe_combine, moe_decode_fused, moe_permute,
               moe_permute_max_tiles, moe_route, moe_route_permute, mxfp4_quant_1x32,
               mxfp4_quant_1x32_chunked, nvfp4_qdq, load)


# moe_route_permute (one launch, one workgroup) takes T * (topk + n_shared) up
# to 1024 pairs.  It routes one token per wavefront of a single CU, so beyond
# about 8 tokens the two launches (one workgroup per token for the routing)
# measured faster.
ROUTE_PERMUTE_MAX_TOKENS = 8

# moe_decode_fused (the whole layer in one launch) takes at most 16 tokens.
FUSED_DECODE_MAX_TOKENS = 16

# Intermediate buffers are kept per batch size for reuse; the least recently
# used sizes beyond this many are released (a serving loop sees many sizes).
MAX_CACHED_BATCH_SIZES = 8


@dataclass
class LayerConfig:
    H: int
    I: int
    E: int                 # routed experts
    n_shared: int          # shared experts (ids E .. E+n_shared-1 in the weight tensors)
    n_group: int
    topk_group: int
    topk: int
    afmt: str              # bf16 | mx | nvfp4 | fp8 (per-token FP8, with FP8 weights)
    wfmt: str              # mx | nvfp4 | fp8
    block_m: int = 16
    renormalize: bool = True
    routed_scale: float = 1.0
    fragment_layout: bool = True   # stream weights from the fragment-major layout
    # one launch (moe_decode_fused) where it applies; off by default: on
    # MI355X its grid barrier and per-item release fences cost more than the
    # kernel boundaries of the chain of calls (measured: T=1 275 us against
    # 57 us, T=8 740 us against 194 us)
    fused_decode: bool = False


class MoELayer:
    """Weights (device tensors):
         w13 [E+n_shared, 2I, H/2] (FP8: [.., H]), w13_scale (E8M0 [.., H/32] |
         E4M3 [.., H/16] | float32 channel scale [E+n_shared, 2I]), w13_ts float32
         [E+n_shared] for NVFP4; w2 / w2_scale / w2_ts likewise with [H, I],
         all in the row-major layout.  With cfg.fragment_layout the codes and
         block scales are rewritten once, here, by fp4_weight_preshuffle (the
         row-major tensors are then no longer referenced).  Pass
         preshuffled=True when the weights already are fragment-major."""

    def __init__(self, cfg: LayerConfig, weights: dict, device="cuda", preshuffled=False):
        load()
        self.cfg = cfg
        self.layout = LAYOUT_FRAGMENT if cfg.fragment_layout else LAYOUT_ROWMAJOR
        if cfg.fragment_layout and not preshuffled:
            weights = dict(weights)
            wf = WFMT[cfg.wfmt]
            for name in ("w13", "w2"):
                sc = None if cfg.wfmt == "fp8" else weights[name + "_scale"]
                c, s = fp4_weight_preshuffle(wf, weights[name], sc)
                weights[name] = c
                if cfg.wfmt != "fp8":
                    weights[name + "_scale"] = s
        self.w = weights
        # Prefill tiles (MXFP4 activations, fragment weights; block_m 128 / 192 /
        # 256 for MXFP4 weights, 192 for FP8 weights) take their activations
        # chunk-major and already in expert order (the stage-1 quantizer writes
        # each token to its pairs' sorted rows), so every tile copy is contiguous.
        self.chunked = (cfg.afmt == "mx" and cfg.fragment_layout and
                        ((cfg.wfmt == "mx" and cfg.block_m in (128, 192, 256)) or
                         (cfg.wfmt == "fp8" and cfg.block_m == 192)))
        # W8A8: per-token FP8 activations (chunk-major) x FP8 weights, 128-row tiles
        self.a8 = cfg.afmt == "fp8"
        if self.a8 and not (cfg.wfmt == "fp8" and cfg.block_m == 128 and cfg.fragment_layout):
            raise ValueError("FP8 activations run with FP8 fragment-major weights and block_m 128")
        # NVFP4 with 64- or 128-row tiles: activations in the f16 operand form
        # of nvfp4_qdq (E2M1 x E4M3 weights decode to f16 with one conversion
        # and one packed multiply per pair); the 128-row tiles stream each
        # weight slice once per 128 rows of its expert and need K % 512 == 0
        n13, n2 = cfg.I, cfg.H
        self.f16a = (cfg.afmt == "nvfp4" and cfg.wfmt == "nvfp4" and cfg.fragment_layout and
                     n13 % 128 == 0 and n2 % 256 == 0 and
                     (cfg.block_m == 64 or
                      (cfg.block_m == 128 and cfg.H % 512 == 0 and cfg.I % 512 == 0)))
        self.device = device
        self._bufs = OrderedDict()
        self.nvfp4_ws = torch.empty(256, dtype=torch.uint8, device=device)
        # the 128-row NVFP4 tiles take their items from a work queue (zero-filled
        # once; every call leaves it so; both stages run in order on one stream)
        self.gemm_queue = (torch.zeros(16, dtype=torch.int32, device=device)
                           if self.f16a and cfg.block_m == 128 else None)
        # the single-launch decode: bf16 activations, fragment-major MXFP4
        # weights, 16-row tiles (its workspace is zero-filled once, here)
        self.fused_ok = (cfg.fused_decode and cfg.afmt == "bf16" and cfg.wfmt == "mx" and
                         cfg.fragment_layout and cfg.block_m == 16 and cfg.H % 128 == 0 and
                         cfg.I % 128 == 0 and cfg.topk <= 16 and cfg.n_shared <= 8 and
                         cfg.E + cfg.n_shared <= 1032)
        self.fused_ws = None
        if self.fused_ok:
            nbytes = load().moe_decode_fused_workspace(cfg.H)
            self.fused_ws = torch.zeros((nbytes + 3) // 4, dtype=torch.int32, device=device)

    def _buffers(self, T):
        if T in self._bufs:
            self._bufs.move_to_end(T)
            return self._bufs[T]
        c = self.cfg
        k = c.topk + c.n_shared
        P = T * k
        dev = self.device
        mt = moe_permute_max_tiles(T, c.topk, c.E, c.n_shared, c.block_m)
        b = dict(
            topk_ids=torch.empty((T, c.topk), dtype=torch.int32, device=dev),
            topk_w=torch.empty((T, c.topk), dtype=torch.float32, device=dev),
            perm=dict(expert_offsets=torch.empty(c.E + c.n_shared + 1, dtype=torch.int32, device=dev),
                      sorted_pairs=torch.empty(P, dtype=torch.int32, device=dev),
                      pair_pos=torch.empty(P, dtype=torch.int32, device=dev),
                      tiles=torch.empty((max(mt, 1), 2), dtype=torch.int32, device=dev),
                      n_tiles=torch.empty(1, dtype=torch.int32, device=dev),
                      n_dropped=torch.empty(1, dtype=torch.int32, device=dev)),
            perm_ws=torch.empty(max(1, load().moe_permute_workspace(T, c.topk, c.E, c.n_shared,
                                                                    c.block_m)),
                                dtype=torch.uint8, device=dev),
            h=torch.empty((P, c.I), dtype=torch.bfloat16, device=dev),
            y=torch.empty((P, c.H), dtype=torch.bfloat16, device=dev),
            out=torch.empty((T, c.H), dtype=torch.bfloat16, device=dev),
        )
        if c.afmt == "mx" and self.chunked:
            b["xq"] = torch.empty((c.H // 128, P, 64), dtype=torch.uint8, device=dev)
            b["xs"] = torch.empty((c.H // 128, P, 4), dtype=torch.uint8, device=dev)
            b["hq"] = torch.empty((c.I // 128, P, 64), dtype=torch.uint8, device=dev)
            b["hs"] = torch.empty((c.I // 128, P, 4), dtype=torch.uint8, device=dev)
        elif c.afmt == "mx":
            b["xq"] = torch.empty((T, c.H // 2), dtype=torch.uint8, device=dev)
            b["xs"] = torch.empty((T, c.H // 32), dtype=torch.uint8, device=dev)
            b["hq"] = torch.empty((P, c.I // 2), dtype=torch.uint8, device=dev)
            b["hs"] = torch.empty((P, c.I // 32), dtype=torch.uint8, device=dev)
        elif c.afmt == "fp8":
            b["xq"] = torch.empty((c.H // 128, T, 128), dtype=torch.uint8, device=dev)
            b["xs"] = torch.empty(T, dtype=torch.float32, device=dev)
            b["hq"] = torch.empty((c.I // 128, P, 128), dtype=torch.uint8, device=dev)
            b["hs"] = torch.empty(P, dtype=torch.float32, device=dev)
        elif c.afmt == "nvfp4":
            dt = torch.float16 if self.f16a else torch.bfloat16
            b["xq"] = torch.empty((T, c.H), dtype=dt, device=dev)
            b["hq"] = torch.empty((P, c.I), dtype=dt, device=dev)
            b["xs"] = torch.empty(1, dtype=torch.float32, device=dev)
            b["hs"] = torch.empty(1, dtype=torch.float32, device=dev)
        self._bufs[T] = b
        while len(self._bufs) > MAX_CACHED_BATCH_SIZES:
            self._bufs.popitem(last=False)
        return b

    def forward(self, x, logits, bias, keep=False, stream=None, events=None):
        """x bf16 [T, H], logits float32 [T, E], bias float32 [E] -> out bf16 [T, H].

        With keep=True returns the dict of every intermediate buffer.  `events`
        (optional) maps a step name ("stage1", "stage2", ...) to a list that
        receives a (start, end) pair of recorded HIP events for that call."""
        c = self.cfg
        tick = _Ticker(events, stream)
        T = x.shape[0]
        k = c.topk + c.n_shared
        b = self._buffers(T)
        if (self.fused_ok and 1 <= T <= FUSED_DECODE_MAX_TOKENS and logits.shape[1] == c.E):
            tick("fused")
            moe_decode_fused(x, logits, bias, self.w["w13"], self.w["w13_scale"], self.w["w2"],
                             self.w["w2_scale"], I=c.I, n_shared=c.n_shared, n_group=c.n_group,
                             topk_group=c.topk_group, topk=c.topk, workspace=self.fused_ws,
                             out=b, renormalize=c.renormalize, routed_scale=c.routed_scale,
                             stream=stream)
            tick(None)
            return b if keep else b["out"]
        # (one launch only when every routed expert is local: the fused call
        # permutes over the same E it routes over)
        if T <= ROUTE_PERMUTE_MAX_TOKENS and T * k <= 1024 and logits.shape[1] == c.E:
            # decode sizes: routing and permutation in one launch
            tick("route_permute")
            _, _, perm = moe_route_permute(logits, bias, c.n_group, c.topk_group, c.topk,
                                           c.n_shared, c.block_m, c.renormalize, c.routed_scale,
                                           topk_ids=b["topk_ids"], topk_w=b["topk_w"],
                                           out=b["perm"], stream=stream)
        else:
            tick("route")
            moe_route(logits, bias, c.n_group, c.topk_group, c.topk, c.renormalize,
                      c.routed_scale, topk_ids=b["topk_ids"], topk_w=b["topk_w"], stream=stream)
            tick("permute")
            perm = moe_permute(b["topk_ids"], c.E, c.n_shared, c.block_m, workspace=b["perm_ws"],
                               out=b["perm"], stream=stream)
        n_rows = perm["expert_offsets"][c.E + c.n_shared:]     # device row count
        wf = WFMT[c.wfmt]
        w = self.w
        if c.afmt != "bf16":
            tick("quant1")
        gather = dict(a_row_gather=perm["sorted_pairs"], gather_div=k)
        a_layout = A_LAYOUT_ROWMAJOR
        if c.afmt == "mx" and self.chunked:
            mxfp4_quant_1x32_chunked(x, row_map=perm["pair_pos"], map_k=k, codes=b["xq"],
                                     scales=b["xs"], stream=stream)
            a1, a1s, af = b["xq"], b["xs"], A_MXFP4
            gather, a_layout = {}, A_LAYOUT_CHUNKED
        elif c.afmt == "mx":
            mxfp4_quant_1x32(x, codes=b["xq"], scales=b["xs"], stream=stream)
            a1, a1s, af = b["xq"], b["xs"], A_MXFP4
        elif c.afmt == "fp8":
            fp8_quant_per_token(x, codes=b["xq"], scales=b["xs"], stream=stream)
            a1, a1s, af = b["xq"], None, A_FP8
            a_layout = A_LAYOUT_CHUNKED
        elif c.afmt == "nvfp4" and self.f16a:
            nvfp4_qdq(x, y_f16=b["xq"], y_f16_scale=b["xs"], no_y=True,
                      workspace=self.nvfp4_ws, stream=stream)
            a1, a1s, af = b["xq"], None, A_F16
        elif c.afmt == "nvfp4":
            nvfp4_qdq(x, y=b["xq"], workspace=self.nvfp4_ws, stream=stream)
            a1, a1s, af = b["xq"], None, A_BF16
        else:
            a1, a1s, af = x, None, A_BF16
        ts13 = w.get("w13_ts") if c.wfmt == "nvfp4" else None
        cs13 = w["w13_scale"] if c.wfmt == "fp8" else None
        tick("stage1")
        # 192-row tiles quantize h for stage 2 in their epilogue (the bf16 h is
        # then written only when the caller keeps the intermediates)
        fused_q = self.chunked and c.block_m == 192
        qkw = dict(out_q=b["hq"], out_q_scale=b["hs"], no_out=not keep) if fused_q else {}
        f16kw = dict(a_f16_scale=b["xs"], work_queue=self.gemm_queue) if self.f16a else {}
        if self.a8:
            f16kw = dict(a_row_scale=b["xs"])
        fp4_grouped_gemm(1, wf, af, w["w13"], None if c.wfmt == "fp8" else w["w13_scale"], a1,
                         perm, c.block_m, a_scale=a1s, w_tensor_scale=ts13, w_channel_scale=cs13,
                         out=b["h"] if (keep or not fused_q) else None, w_layout=self.layout,
                         a_layout=a_layout, stream=stream, **qkw, **gather, **f16kw)
        if c.afmt != "bf16" and not fused_q:
            tick("quant2")
        if fused_q:
            a2, a2s = b["hq"], b["hs"]
        elif c.afmt == "mx" and self.chunked:
            mxfp4_quant_1x32_chunked(b["h"], row_count=n_rows, codes=b["hq"], scales=b["hs"],
                                     stream=stream)
            a2, a2s = b["hq"], b["hs"]
        elif c.afmt == "mx":
            mxfp4_quant_1x32(b["h"], row_count=n_rows, codes=b["hq"], scales=b["hs"],
                             stream=stream)
            a2, a2s = b["hq"], b["hs"]
        elif c.afmt == "fp8":
            fp8_quant_per_token(b["h"], row_count=n_rows, codes=b["hq"], scales=b["hs"],
                                stream=stream)
            a2, a2s = b["hq"], None
        elif c.afmt == "nvfp4" and self.f16a:
            nvfp4_qdq(b["h"], row_count=n_rows, y_f16=b["hq"], y_f16_scale=b["hs"], no_y=True,
                      workspace=self.nvfp4_ws, stream=stream)
            a2, a2s = b["hq"], None
        elif c.afmt == "nvfp4":
            nvfp4_qdq(b["h"], row_count=n_rows, y=b["hq"], workspace=self.nvfp4_ws,
                      stream=stream)
            a2, a2s = b["hq"], None
        else:
            a2, a2s = b["h"], None
        ts2 = w.get("w2_ts") if c.wfmt == "nvfp4" else None
        cs2 = w["w2_scale"] if c.wfmt == "fp8" else None
        tick("stage2")
        f16kw = dict(a_f16_scale=b["hs"], work_queue=self.gemm_queue) if self.f16a else {}
        if self.a8:
            f16kw = dict(a_row_scale=b["hs"])
        fp4_grouped_gemm(2, wf, af, w["w2"], None if c.wfmt == "fp8" else w["w2_scale"], a2, perm,
                         c.block_m, a_scale=a2s, w_tensor_scale=ts2, w_channel_scale=cs2,
                         out=b["y"], w_layout=self.layout, a_layout=a_layout, stream=stream,
                         **f16kw)
        tick("combine")
        moe_combine(b["y"], perm["pair_pos"], b["topk_w"], c.topk, c.n_shared, out=b["out"],
                    stream=stream)
        tick(None)
        return b if keep else b["out"]


class _Ticker:
    """Records a HIP event between consecutive steps when `events` is given."""

    def __init__(self, events, stream):
        self.events = events
        self.stream = stream
        self.name = None
        self.start = None

    def __call__(self, name):
        if self.events is None:
            return
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(self.stream if self.stream is not None else torch.cuda.current_stream())
        if self.name is not None:
            self.events.setdefault(self.name, []).append((self.start, ev))
        self.name, self.start = name, ev
