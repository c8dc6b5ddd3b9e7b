#!/usr/bin/env python3
"""Benchmark of the block-scaled FP4 routed-expert MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline: the decode MoE layer of the DeepSeek-V3 / Kimi K2 shape (hidden
7168, expert intermediate 2048, 384 routed experts top-8 in 8 groups keeping
4, one shared expert), MXFP4 weights (E2M1 + E8M0 per 1x32) decoded to bf16
inside the GEMM tile, bf16 activations, T = 8 tokens.  One step is one pass
of the whole layer (route, permute, gate/up GEMM + SiLU*up, down GEMM,
combine) over one batch.  `value` is the layer's weight-streaming rate:
algorithmic bytes (weights of every expert the batch touches, plus the
token activations in and out and the router logits) per second, inputs
resident in HBM.  Batches rotate over 16 seeded routing draws so successive
steps touch different experts and the last-level cache cannot hold the
working set.

Also reported on the same line:
  decode_sweep  the same layer at T = 1 and 64
  decode_expert_scaling
                each decode GEMM stage alone against the number of touched
                experts (one row each), the items-per-compute-unit picture
  prefill       T = 8192, uniform routing, MXFP4 activations and the gfx950
                scaled FP4 x FP4 MFMA: TFLOP/s = 88,080,384 FLOP per
                (token, expert) pair
  roofline      the dominant kernel (stage-1 gate/up GEMM) timed with HIP
                events on its launch stream, against the 8 TB/s HBM peak
  cpu_baseline  the CPU oracle (NumPy float64) on a bounded sample

Only one GPU is used: --gpus above 1 exits with a message.
"""

import argparse
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MXFP4_PEAK_TFLOPS = 10100.0    # MI355X dense MXFP4 matrix peak
BYTES_W13 = 4096 * 3584 + 4096 * 224     # one expert's fused gate/up weight, MXFP4
BYTES_W2 = 7168 * 1024 + 7168 * 64       # one expert's down weight, MXFP4
FLOP_PER_PAIR = 2 * 7168 * 4096 + 2 * 2048 * 7168
BYTES_NV_W13 = 4096 * 3584 + 4096 * 448   # one expert's fused gate/up weight, NVFP4 (E4M3 per 16)
BYTES_NV_W2 = 7168 * 1024 + 7168 * 128
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 matrix peak (the FP4 x FP8 scaled MFMA rate)
FP8_BLOCK_M = 192              # FP8-weight layer: 192-row tiles on the scaled MFMA
METRIC = "FP4 MoE layer TFLOP/s (prefill) + weight GB/s (decode) on 1 MI355X"
N_ROTATE = 16

# HBM traffic of the roofline kernel on the T=8 decode workload, from two
# rocprofv3 counter passes (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch,
# mean over the rotated routing draws), each scaled by what that counter reads
# for a plain 1 GiB copy (FETCH_SIZE reads half the bytes: x1.9999; WRITE_SIZE
# x1.0).  Reported only while the kernel's sources hash to what they were when
# the counters were taken; otherwise traffic is null.  Keyed by kernel.
ROOFLINE_COUNTERS = {
    "stage1": dict(
        tokens=8, fetch_kib=378988.3, write_kib=288.0, fetch_scale=1.9999, write_scale=1.0,
        sources=("block_scaled_fp4_moe_amd/csrc/gemm_dq.hip",
                 "block_scaled_fp4_moe_amd/csrc/dq_item.h",
                 "block_scaled_fp4_moe_amd/csrc/gemm_common.h",
                 "block_scaled_fp4_moe_amd/csrc/common.h"),
        sha256=("237f7aabeb9862f75362261cdfd07d2873ad244bcaf1a0bacca908f035546f26",
                "b093c60db7909994542252865dae0a72a06224d6e2ba49d207411efd98846d82",
                "d0ae32a13fb9a774a315dbdf9c73817cc42ca9f2669bd57489ece84cb5d84a2d",
                "3af844087c30bbbc3272119b6ca934e877d90b1159a2b45ad9077007c79fd1c0")),
}


def roofline_traffic(kernel, tokens):
    """Counter-derived HBM bytes per launch of `kernel`, or None if stale or absent."""
    import hashlib
    c = ROOFLINE_COUNTERS.get(kernel)
    if c is None or tokens != c["tokens"]:
        return None
    root = os.path.dirname(os.path.abspath(__file__))
    for rel, want in zip(c["sources"], c["sha256"]):
        with open(os.path.join(root, rel), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != want:
                return None
    return int((c["fetch_kib"] * c["fetch_scale"] + c["write_kib"] * c["write_scale"]) * 1024)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--tokens", type=int, default=8, help="decode batch of the headline")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the NVFP4 layer and the FP8 conversion / FP8 layer measurements")
    ap.add_argument("--extra", default="nvfp4,fp8,dense",
                    help="comma-separated subset of the extra workloads to measure "
                         "(nvfp4, fp8, dense)")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 1 GiB device-to-device copy (counter calibration)")
    args = ap.parse_args()
    args.extra = [x.strip() for x in args.extra.split(",") if x.strip()]
    bad = [x for x in args.extra if x not in ("nvfp4", "fp8", "dense")]
    if bad:
        ap.error(f"--extra: unknown workload(s) {bad} (choose from nvfp4, fp8, dense)")
    return args


def log(args, *a):
    if not args.quiet:
        print("[bench]", *a, file=sys.stderr, flush=True)


def make_weights(w, torch):
    """All 385 experts' MXFP4 weights, generated by the seeded synth streams."""
    Et = w.E + w.n_shared
    H, I = w.H, w.I
    dev = dict(w13=torch.empty((Et, 2 * I, H // 2), dtype=torch.uint8, device="cuda"),
               w13_scale=torch.empty((Et, 2 * I, H // 32), dtype=torch.uint8, device="cuda"),
               w2=torch.empty((Et, H, I // 2), dtype=torch.uint8, device="cuda"),
               w2_scale=torch.empty((Et, H, I // 32), dtype=torch.uint8, device="cuda"))
    import synth

    def gen(e):
        return e, synth.expert_mx(w, e, 13), synth.expert_mx(w, e, 2)

    with ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0))))) as ex:
        for e, (c13, s13), (c2, s2) in ex.map(gen, range(Et)):
            dev["w13"][e].copy_(torch.from_numpy(c13))
            dev["w13_scale"][e].copy_(torch.from_numpy(s13))
            dev["w2"][e].copy_(torch.from_numpy(c2))
            dev["w2_scale"][e].copy_(torch.from_numpy(s2))
    # static weights are rewritten once into the fragment-major layout
    import block_scaled_fp4_moe_amd as fm
    for name in ("w13", "w2"):
        c, s = fm.fp4_weight_preshuffle(fm.W_MXFP4, dev[name], dev[name + "_scale"])
        dev[name], dev[name + "_scale"] = c, s
    return dev


def batch_inputs(w, T, seed, torch):
    import synth
    x = torch.from_numpy(synth.activations(w, T, seed).view(np.int16)).cuda().view(torch.bfloat16)
    logits = torch.from_numpy(synth.router_logits(w, T, seed)).cuda()
    return x, logits


def touched_experts(layer, T):
    """Distinct experts (routed + shared) with rows after the last forward (device read)."""
    b = layer._bufs[T]
    offs = b["perm"]["expert_offsets"].cpu().numpy()
    return int(np.count_nonzero(np.diff(offs)))


def time_layer(layer, batches, bias, steps, warmup, torch, with_events=True):
    """Time `steps` layer passes after `warmup` untimed ones; returns dict."""
    T = batches[0][0].shape[0]
    n = len(batches)
    # bytes per batch (untimed accounting pass)
    experts = []
    for x, lg in batches:
        layer.forward(x, lg, bias)
        torch.cuda.synchronize()
        experts.append(touched_experts(layer, T))
    for s in range(warmup):
        x, lg = batches[s % n]
        layer.forward(x, lg, bias)
    # timed pass 1: the layer alone (no per-kernel events inside the steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    touched = 0
    for s in range(steps):
        x, lg = batches[s % n]
        layer.forward(x, lg, bias)
        touched += experts[s % n]
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(end)
    # timed pass 2: the same steps with a HIP event pair around every call,
    # recorded on the stream the kernels are launched on
    per_kernel = {}
    if with_events:
        events = {}
        for s in range(steps):
            x, lg = batches[s % n]
            layer.forward(x, lg, bias, events=events)
        torch.cuda.synchronize()
        for name, pairs in events.items():
            per_kernel[name] = sum(a.elapsed_time(b) for a, b in pairs) / len(pairs)
    # timed pass 3: one event pair around each step, for the spread of step
    # times; pass 4 ("cold"): the same after reading a 1 GiB buffer before
    # each step (clean lines only), so that no weight byte is left in the
    # L2 or the last-level cache
    dist = {}
    if with_events:
        flush = torch.ones(1 << 27, dtype=torch.int64, device="cuda")
        sink = torch.empty(1, dtype=torch.int64, device="cuda")
        for mode in ("rotated", "cold"):
            pairs = []
            for s in range(steps):
                x, lg = batches[s % n]
                if mode == "cold":
                    torch.sum(flush, dim=0, keepdim=True, out=sink)
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                layer.forward(x, lg, bias)
                b.record()
                pairs.append((a, b, experts[s % n]))
            torch.cuda.synchronize()
            ms = np.array([a.elapsed_time(b) for a, b, _ in pairs])
            dist[mode] = dict(p10=float(np.percentile(ms, 10)), p50=float(np.percentile(ms, 50)),
                              p90=float(np.percentile(ms, 90)),
                              touched=float(np.mean([t for _, _, t in pairs])))
        del flush, sink
    return dict(ms_per_step=gpu_ms / steps, wall_s=wall, touched_per_step=touched / steps,
                per_kernel_ms=per_kernel, experts_per_batch=experts, dist=dist)


def decode_bytes(cfg, T, touched):
    return touched * (BYTES_W13 + BYTES_W2) + 2 * T * cfg.H * 2 + T * cfg.E * 4


def run_decode(fm, w, dev_w, T, steps, warmup, torch, args, fused=False):
    """The decode layer at T tokens: the chain of calls, or with `fused` the
    single launch (moe_decode_fused)."""
    import synth
    cfg = fm.LayerConfig(H=w.H, I=w.I, E=w.E, n_shared=w.n_shared, n_group=w.n_group,
                         topk_group=w.topk_group, topk=w.topk, afmt="bf16", wfmt="mx", block_m=16,
                         fused_decode=fused)
    layer = fm.MoELayer(cfg, dev_w, preshuffled=True)
    bias = torch.from_numpy(synth.router_bias(w)).cuda()
    batches = [batch_inputs(w, T, 1000 + i, torch) for i in range(N_ROTATE)]
    r = time_layer(layer, batches, bias, steps, warmup, torch)
    step_bytes = decode_bytes(cfg, T, r["touched_per_step"])
    r["gbs"] = step_bytes / (r["ms_per_step"] * 1e-3) / 1e9
    r["bytes_per_step"] = step_bytes
    # dominant kernel: the single-launch layer (its algorithmic bytes per
    # launch are the step's: touched experts' weights + x in + out + logits),
    # else the stage-1 gate/up GEMM of the chain (touched experts x W13 bytes
    # + gathered activations in + h out)
    k = w.topk + w.n_shared
    if "fused" in r["per_kernel_ms"]:
        rk, rk_bytes, rk_ms = "fused", step_bytes, r["per_kernel_ms"]["fused"]
    else:
        rk = "stage1"
        rk_bytes = r["touched_per_step"] * BYTES_W13 + T * cfg.H * 2 + T * k * cfg.I * 2
        rk_ms = r["per_kernel_ms"]["stage1"]
    r["roofline_kernel"] = dict(name=rk, ms=rk_ms, bytes=rk_bytes,
                                gbs=rk_bytes / (rk_ms * 1e-3) / 1e9)
    # step-time spread (one event pair per step) and the cold-cache figure
    r["spread"] = {}
    for mode, d in r["dist"].items():
        b = decode_bytes(cfg, T, d["touched"])
        r["spread"][mode] = dict(us_p10=round(d["p10"] * 1e3, 1), us_p50=round(d["p50"] * 1e3, 1),
                                 us_p90=round(d["p90"] * 1e3, 1),
                                 gbs_p50=round(b / (d["p50"] * 1e-3) / 1e9, 1))
    log(args, f"decode T={T}: {r['ms_per_step']*1e3:.1f} us/step, {r['gbs']:.0f} GB/s, "
              f"{r['touched_per_step']:.1f} experts/step, kernels(us)="
              + json.dumps({k2: round(v * 1e3, 1) for k2, v in r['per_kernel_ms'].items()})
              + ", step spread " + json.dumps(r["spread"]))
    return r


def run_expert_scaling(fm, w, dev_w, torch, args, counts=(1, 2, 4, 8, 9, 12, 16, 32)):
    """Each decode GEMM stage alone with one row on each of n routed experts
    (n = 9 is the T=1 layer: 8 routed + the shared expert), 32 disjoint expert
    sets rotated so that no weight byte is reused from the caches.  Shows how
    the time follows the bytes each compute unit streams: the work items
    (16-row tile x 32 output columns in stage 1, x 64 in stage 2) are spread
    over the 256 compute units, and one unit alone streams about 20-25 GB/s."""
    H, I, E = w.H, w.I, w.E
    x = batch_inputs(w, 32, 77, torch)[0]
    h = x[:, :I].contiguous()
    hb = torch.empty(32, I, dtype=torch.bfloat16, device="cuda")
    yb = torch.empty(32, H, dtype=torch.bfloat16, device="cuda")

    def timed(calls, reps=3):
        for c in calls[:4]:
            c()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for c in calls:
                c()
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) * 1e3 / len(calls)
            best = us if best is None else min(best, us)
        return best

    rows = []
    for n in counts:
        perms = []
        for r in range(32):
            ids = torch.tensor([[(r * 12 + j * 41) % E] for j in range(n)], dtype=torch.int32,
                               device="cuda")
            perms.append(fm.moe_permute(ids, E, 0, 16))
        s1 = [lambda p=p: fm.fp4_grouped_gemm(1, fm.W_MXFP4, fm.A_BF16, dev_w["w13"],
                                              dev_w["w13_scale"], x, p, 16,
                                              a_row_gather=p["sorted_pairs"], gather_div=1,
                                              out=hb, w_layout=fm.LAYOUT_FRAGMENT) for p in perms]
        s2 = [lambda p=p: fm.fp4_grouped_gemm(2, fm.W_MXFP4, fm.A_BF16, dev_w["w2"],
                                              dev_w["w2_scale"], h, p, 16, out=yb,
                                              w_layout=fm.LAYOUT_FRAGMENT) for p in perms]
        t1, t2 = timed(s1), timed(s2)
        rows.append(dict(experts=n, stage1_us=round(t1, 2),
                         stage1_gbs=round(n * BYTES_W13 / (t1 * 1e3), 1),
                         stage1_items_per_cu=round(n * (I // 32) / 256, 3),
                         stage2_us=round(t2, 2),
                         stage2_gbs=round(n * BYTES_W2 / (t2 * 1e3), 1),
                         stage2_items_per_cu=round(n * (H // 64) / 256, 3)))
        log(args, "expert scaling " + json.dumps(rows[-1]))
    return rows


EP_RANKS = 8


def run_ep_share(fm, w, dev_w, T, steps, warmup, torch, args):
    """One rank's share of the decode layer under expert parallelism over 8
    GPUs: the 48 routed experts [0, 48) plus the shared expert on this GPU, the
    router over all 384 experts, pairs routed elsewhere dropped by the
    permutation (no exchange is timed: one GPU only)."""
    import synth
    E_loc = w.E // EP_RANKS
    idx = torch.tensor(list(range(E_loc)) + list(range(w.E, w.E + w.n_shared)), device="cuda")
    loc_w = {k: v.index_select(0, idx).contiguous() for k, v in dev_w.items()}
    cfg = fm.LayerConfig(H=w.H, I=w.I, E=E_loc, n_shared=w.n_shared, n_group=w.n_group,
                         topk_group=w.topk_group, topk=w.topk, afmt="bf16", wfmt="mx", block_m=16)
    layer = fm.MoELayer(cfg, loc_w, preshuffled=True)
    bias = torch.from_numpy(synth.router_bias(w)).cuda()
    batches = [batch_inputs(w, T, 1000 + i, torch) for i in range(N_ROTATE)]
    r = time_layer(layer, batches, bias, steps, warmup, torch)
    step_bytes = (r["touched_per_step"] * (BYTES_W13 + BYTES_W2) + 2 * T * w.H * 2 +
                  T * w.E * 4)
    gbs = step_bytes / (r["ms_per_step"] * 1e-3) / 1e9
    log(args, f"EP{EP_RANKS} share decode T={T}: {r['ms_per_step']*1e3:.1f} us/step, "
              f"{gbs:.0f} GB/s, {r['touched_per_step']:.1f} local experts/step")
    del layer, loc_w
    return dict(us_per_step=round(r["ms_per_step"] * 1e3, 2), gbs=round(gbs, 1),
                frac=round(gbs / HBM_PEAK_GBS, 4),
                local_experts_per_step=round(r["touched_per_step"], 2),
                kernels_us={k: round(v * 1e3, 2) for k, v in r["per_kernel_ms"].items()},
                workload=f"decode T={T}, one of {EP_RANKS} expert-parallel ranks: routed experts "
                         f"[0, {E_loc}) + the shared expert local, routing over all {w.E}")


def run_prefill(fm, dev_w, steps, torch, args):
    import synth
    w = synth.WORKLOADS["prefill"]
    cfg = fm.LayerConfig(H=w.H, I=w.I, E=w.E, n_shared=w.n_shared, n_group=w.n_group,
                         topk_group=w.topk_group, topk=w.topk, afmt="mx", wfmt="mx", block_m=192)
    layer = fm.MoELayer(cfg, dev_w, preshuffled=True)
    bias = torch.from_numpy(synth.router_bias(w)).cuda()
    batches = [batch_inputs(w, w.T, 2000 + i, torch) for i in range(2)]
    r = time_layer(layer, batches, bias, steps, 2, torch)
    pairs = w.T * (w.topk + w.n_shared)
    r["tflops"] = FLOP_PER_PAIR * pairs / (r["ms_per_step"] * 1e-3) / 1e12
    log(args, f"prefill T={w.T}: {r['ms_per_step']:.3f} ms/step, {r['tflops']:.0f} TFLOP/s, kernels(ms)="
              + json.dumps({k2: round(v, 3) for k2, v in r['per_kernel_ms'].items()}))
    return r


def run_skewed_mx(fm, dev_w, steps, torch, args):
    """Skewed-routing prefill: T=16384, expert popularity Zipf(1.1) over 384
    experts (Gumbel-top-k logits), MXFP4 activations x MXFP4 weights on the
    scaled FP4 MFMA, 192-row tiles (the prefill kernels)."""
    import synth
    w = synth.WORKLOADS["skewed"]
    cfg = fm.LayerConfig(H=w.H, I=w.I, E=w.E, n_shared=w.n_shared, n_group=w.n_group,
                         topk_group=w.topk_group, topk=w.topk, afmt="mx", wfmt="mx", block_m=192)
    layer = fm.MoELayer(cfg, dev_w, preshuffled=True)
    bias = torch.from_numpy(synth.router_bias(w)).cuda()
    batches = [batch_inputs(w, w.T, 5000, torch)]
    r = time_layer(layer, batches, bias, steps, 2, torch)
    pairs = w.T * (w.topk + w.n_shared)
    tflops = FLOP_PER_PAIR * pairs / (r["ms_per_step"] * 1e-3) / 1e12
    offs = layer._bufs[w.T]["perm"]["expert_offsets"].cpu().numpy()
    counts = np.diff(offs)[:w.E]
    log(args, f"skewed mx prefill T={w.T}: {r['ms_per_step']:.3f} ms/step, {tflops:.0f} TFLOP/s, "
              f"rows per routed expert max {counts.max()} median {int(np.median(counts))} "
              f"min {counts.min()}, kernels(ms)="
              + json.dumps({k2: round(v, 3) for k2, v in r['per_kernel_ms'].items()}))
    del layer
    torch.cuda.empty_cache()
    return dict(tflops=round(tflops, 1), ms_per_step=round(r["ms_per_step"], 3),
                frac=round(tflops / MXFP4_PEAK_TFLOPS, 4),
                kernels_ms={k: round(v, 4) for k, v in r["per_kernel_ms"].items()},
                rows_per_routed_expert=dict(max=int(counts.max()), median=float(np.median(counts)),
                                            min=int(counts.min()),
                                            empty=int(np.count_nonzero(counts == 0))),
                workload=f"skewed prefill MoE layer, T={w.T}, Zipf(1.1) expert popularity over "
                         f"{w.E} experts + 1 shared, MXFP4 activations (mxfp4_quant_1x32) x "
                         "MXFP4 weights, gfx950 scaled MFMA, block_m 192")


def gpu_nvfp4_weights(w, torch, seed=4):
    """NVFP4 weights of all experts drawn on the GPU (seeded torch generator) with
    the same distributions as synth.expert_nvfp4: uniform E2M1 bytes, E4M3
    scales = RNE(|N(0,1)|), tensor scale U(0.01, 0.02) per expert and projection."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    Et = w.E + w.n_shared
    out = {}
    for name, (N, K) in (("w13", (2 * w.I, w.H)), ("w2", (w.H, w.I))):
        out[name] = torch.randint(0, 256, (Et, N, K // 2), dtype=torch.uint8, device="cuda",
                                  generator=g)
        sc = torch.randn((Et, N, K // 16), device="cuda", generator=g).abs_()
        out[name + "_scale"] = sc.to(torch.float8_e4m3fn).view(torch.uint8)
        del sc
        out[name + "_ts"] = torch.rand(Et, device="cuda", generator=g) * 0.01 + 0.01
    return out


def gpu_spanned_mx_weights(w, torch, seed=5):
    """MXFP4 weights of all experts drawn on the GPU with the row-scale recipe of
    synth.spanned_scales: top code 127+U{-4..0}, span U{1..9} binades, one block
    at each end of the span, the rest uniform in between; codes uniform bytes.
    Every tensor is drawn for all experts at once (a handful of launches per
    tensor, no per-expert loop)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    Et = w.E + w.n_shared
    out = {}
    for name, (N, K) in (("w13", (2 * w.I, w.H)), ("w2", (w.H, w.I))):
        out[name] = torch.randint(0, 256, (Et, N, K // 2), dtype=torch.uint8, device="cuda",
                                  generator=g)
        nb = K // 32
        i32 = dict(dtype=torch.int32, device="cuda", generator=g)
        top = 127 + torch.randint(-4, 1, (Et, N, 1), **i32)
        span = torch.randint(1, 10, (Et, N, 1), **i32)
        p0 = torch.randint(0, nb, (Et, N, 1), **i32)
        p1 = (p0 + 1 + torch.randint(0, nb - 1, (Et, N, 1), **i32)) % nb
        col = torch.arange(nb, dtype=torch.int32, device="cuda").view(1, 1, nb)
        s_ = top - torch.randint(0, 1 << 30, (Et, N, nb), **i32) % (span + 1)
        s_ = torch.where(col == p0, top, s_)
        s_ = torch.where(col == p1, top - span, s_)
        out[name + "_scale"] = s_.to(torch.uint8)
        del top, span, p0, p1, s_
    return out


def run_nvfp4(fm, steps, torch, args):
    """NVFP4 emulation layer, T=2048: E4M3-per-16 weights decoded in-tile, activations
    QDQ'd before each GEMM; weight GB/s against the HBM peak."""
    import synth
    w = synth.WORKLOADS["nvfp4"]
    dev_w = gpu_nvfp4_weights(w, torch)
    cfg = fm.LayerConfig(H=w.H, I=w.I, E=w.E, n_shared=w.n_shared, n_group=w.n_group,
                         topk_group=w.topk_group, topk=w.topk, afmt="nvfp4", wfmt="nvfp4",
                         block_m=128)
    layer = fm.MoELayer(cfg, dev_w)
    del dev_w
    bias = torch.from_numpy(synth.router_bias(w)).cuda()
    batches = [batch_inputs(w, w.T, 4000 + i, torch) for i in range(2)]
    r = time_layer(layer, batches, bias, steps, 2, torch)
    step_bytes = (r["touched_per_step"] * (BYTES_NV_W13 + BYTES_NV_W2) + 2 * w.T * w.H * 2
                  + w.T * w.E * 4)
    gbs = step_bytes / (r["ms_per_step"] * 1e-3) / 1e9
    log(args, f"nvfp4 T={w.T}: {r['ms_per_step']:.3f} ms/step, {gbs:.0f} GB/s, "
              f"{r['touched_per_step']:.0f} experts")
    del layer
    torch.cuda.empty_cache()
    return dict(gbs=round(gbs, 1), ms_per_step=round(r["ms_per_step"], 4),
                frac=round(gbs / HBM_PEAK_GBS, 4),
                experts_per_step=round(r["touched_per_step"], 1),
                kernels_ms={k: round(v, 4) for k, v in r["per_kernel_ms"].items()},
                workload=f"NVFP4 emulation MoE layer, T={w.T}, 384 experts top-8, E4M3 per-16 "
                         "weight scales + fp32 tensor scale decoded to f16 in-tile (128-row "
                         "tiles), activation QDQ before each GEMM; weights drawn on the GPU")


def run_fp8(fm, steps, torch, args):
    """Skewed-routing workload: exact MXFP4 -> FP8 per-channel conversion of all
    experts (HBM-bound), then the FP8-weight layer at T=16384 (Zipf routing)."""
    import synth
    w = synth.WORKLOADS["skewed"]
    mx = gpu_spanned_mx_weights(w, torch)
    Et = w.E + w.n_shared
    res = {}
    conv = {}
    for name, (N, K) in (("w13", (2 * w.I, w.H)), ("w2", (w.H, w.I))):
        codes = mx[name].view(Et * N, K // 2)
        scales = mx[name + "_scale"].view(Et * N, K // 32)
        outs = fm.mxfp4_to_fp8_channel(codes, scales)            # warm-up and output buffers
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        reps = 3
        a.record()
        for _ in range(reps):
            fm.mxfp4_to_fp8_channel(codes, scales, *outs)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        nbytes = codes.numel() + scales.numel() + outs[0].numel() + 4 * Et * N + Et * N
        conv[name] = dict(ms=ms, bytes=nbytes, n_inexact=int(outs[3].item()),
                          fp8=outs[0].view(Et, N, K), scale=outs[1].view(Et, N))
    del mx
    torch.cuda.empty_cache()
    ms = conv["w13"]["ms"] + conv["w2"]["ms"]
    nbytes = conv["w13"]["bytes"] + conv["w2"]["bytes"]
    res["convert"] = dict(gbs=round(nbytes / (ms * 1e-3) / 1e9, 1), ms=round(ms, 4),
                          frac=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          bytes=int(nbytes),
                          inexact_rows=conv["w13"]["n_inexact"] + conv["w2"]["n_inexact"],
                          workload=f"mxfp4_to_fp8_channel over all {Et} experts' gate/up "
                                   "(4096x7168) and down (7168x2048) weights, row scale spans "
                                   "U{1..9} binades")
    log(args, f"fp8 conversion: {ms:.3f} ms, {res['convert']['gbs']:.0f} GB/s")
    dev_w = dict(w13=conv["w13"]["fp8"], w13_scale=conv["w13"]["scale"],
                 w2=conv["w2"]["fp8"], w2_scale=conv["w2"]["scale"])
    del conv
    cfg = fm.LayerConfig(H=w.H, I=w.I, E=w.E, n_shared=w.n_shared, n_group=w.n_group,
                         topk_group=w.topk_group, topk=w.topk, afmt="mx", wfmt="fp8",
                         block_m=FP8_BLOCK_M)
    layer = fm.MoELayer(cfg, dev_w)
    del dev_w
    bias = torch.from_numpy(synth.router_bias(w)).cuda()
    batches = [batch_inputs(w, w.T, 5000, torch)]
    r = time_layer(layer, batches, bias, steps, 1, torch)
    tflops = FLOP_PER_PAIR * w.T * (w.topk + w.n_shared) / (r["ms_per_step"] * 1e-3) / 1e12
    log(args, f"fp8 layer T={w.T}: {r['ms_per_step']:.3f} ms/step, {tflops:.0f} TFLOP/s")
    res["layer"] = dict(tflops=round(tflops, 1), ms_per_step=round(r["ms_per_step"], 3),
                        frac_of_fp8_peak=round(tflops / FP8_PEAK_TFLOPS, 4),
                        kernels_ms={k: round(v, 4) for k, v in r["per_kernel_ms"].items()},
                        workload=f"FP8-weight MoE layer, T={w.T}, Zipf(1.1) routing, converted "
                                 "E4M3 weights x MXFP4 activations on the gfx950 scaled MFMA "
                                 f"(FP4 x FP8, block_m {FP8_BLOCK_M})")
    # W8A8: the same converted experts with dynamic per-token FP8 activations
    cfg8 = fm.LayerConfig(H=w.H, I=w.I, E=w.E, n_shared=w.n_shared, n_group=w.n_group,
                          topk_group=w.topk_group, topk=w.topk, afmt="fp8", wfmt="fp8",
                          block_m=128)
    layer8 = fm.MoELayer(cfg8, layer.w, preshuffled=True)
    del layer
    torch.cuda.empty_cache()
    r = time_layer(layer8, batches, bias, steps, 1, torch)
    tflops = FLOP_PER_PAIR * w.T * (w.topk + w.n_shared) / (r["ms_per_step"] * 1e-3) / 1e12
    log(args, f"w8a8 layer T={w.T}: {r['ms_per_step']:.3f} ms/step, {tflops:.0f} TFLOP/s, "
              "kernels(ms)=" + json.dumps({k2: round(v, 3) for k2, v in r['per_kernel_ms'].items()}))
    res["w8a8_layer"] = dict(tflops=round(tflops, 1), ms_per_step=round(r["ms_per_step"], 3),
                             frac_of_fp8_peak=round(tflops / FP8_PEAK_TFLOPS, 4),
                             kernels_ms={k: round(v, 4) for k, v in r["per_kernel_ms"].items()},
                             workload=f"W8A8 MoE layer, T={w.T}, Zipf(1.1) routing, converted "
                                      "E4M3 weights (per-channel scales) x dynamic per-token FP8 "
                                      "activations (fp8_quant_per_token) on the gfx950 scaled "
                                      "MFMA (FP8 x FP8, block_m 128)")
    del layer8
    torch.cuda.empty_cache()
    return res


DENSE_SHAPE = (16384, 7168, 7168)   # M tokens, N outputs, K inputs


def run_dense(fm, steps, torch, args):
    """Dense MXFP4 x MXFP4 linear (mxfp4_linear) at the hidden width: the
    activation quantization (chunk-major) and the GEMM, timed apart."""
    M, N, K = DENSE_SHAPE
    g = torch.Generator(device="cuda")
    g.manual_seed(6)
    codes = torch.randint(0, 256, (1, N, K // 2), dtype=torch.uint8, device="cuda", generator=g)
    scales = (119 + torch.randint(0, 7, (1, N, K // 32), dtype=torch.int32, device="cuda",
                                  generator=g)).to(torch.uint8)
    wc, ws = fm.fp4_weight_preshuffle(fm.WFMT["mx"], codes, scales)
    del codes, scales
    x = torch.randn((M, K), dtype=torch.float32, device="cuda", generator=g).to(torch.bfloat16)
    qc = torch.empty((K // 128, M, 64), dtype=torch.uint8, device="cuda")
    qs = torch.empty((K // 128, M, 4), dtype=torch.uint8, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def quant():
        fm.mxfp4_quant_1x32_chunked(x, codes=qc, scales=qs)

    def gemm():
        fm.mxfp4_linear(qc, qs, wc[0], ws[0], a_layout=fm.A_LAYOUT_CHUNKED, out=out)

    res = {}
    for name, f in (("quant", quant), ("gemm", gemm)):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            f()
        b.record()
        torch.cuda.synchronize()
        res[name] = a.elapsed_time(b) / steps
    flop = 2.0 * M * N * K
    tf = flop / (res["gemm"] * 1e-3) / 1e12
    tf_all = flop / ((res["gemm"] + res["quant"]) * 1e-3) / 1e12
    log(args, f"dense mxfp4_linear {M}x{N}x{K}: gemm {res['gemm']:.3f} ms = {tf:.0f} TFLOP/s, "
              f"with activation quantization {tf_all:.0f} TFLOP/s")
    return dict(tflops=round(tf, 1), frac=round(tf / MXFP4_PEAK_TFLOPS, 4),
                gemm_ms=round(res["gemm"], 4), quant_ms=round(res["quant"], 4),
                tflops_with_quant=round(tf_all, 1),
                workload=f"dense MXFP4 linear, M={M} N={N} K={K}: mxfp4_quant_1x32_chunked "
                         "activations x fragment-major MXFP4 weight, 192x512 scaled-MFMA tiles")


def blas_threads():
    """Threads of the BLAS library NumPy calls (threadpoolctl), or None."""
    try:
        import threadpoolctl
        info = [d for d in threadpoolctl.threadpool_info() if d.get("user_api") == "blas"]
        return int(info[0]["num_threads"]) if info else None
    except Exception:
        return None


def _oracle_layer_timed(wl, T, seed, afmt, wfmt, tokens=None):
    """Time the oracle layer (routing included) on the tokens `tokens` of a seeded
    batch of T tokens of workload wl; weight generation is not timed.
    Returns (seconds, pairs, distinct experts read)."""
    import synth
    from oracle import layer as OL
    from oracle import route as OR
    logits = synth.router_logits(wl, T, seed)
    bias = synth.router_bias(wl)
    xb = synth.activations(wl, T, seed)
    if tokens is not None:
        logits, xb = logits[tokens], xb[tokens]
    ids, _ = OR.moe_route(logits, bias, wl.n_group, wl.topk_group, wl.topk)
    experts = sorted(set(ids.reshape(-1).tolist()) | set(range(wl.E, wl.E + wl.n_shared)))
    names = ("w13", "w13_scale", "w2", "w2_scale") + (("w13_ts", "w2_ts") if wfmt == "nvfp4"
                                                      else ())
    np_w = {k: {} for k in names}
    for e in experts:
        if wfmt == "nvfp4":
            np_w["w13"][e], np_w["w13_scale"][e], np_w["w13_ts"][e] = synth.expert_nvfp4(wl, e, 13)
            np_w["w2"][e], np_w["w2_scale"][e], np_w["w2_ts"][e] = synth.expert_nvfp4(wl, e, 2)
        else:
            np_w["w13"][e], np_w["w13_scale"][e] = synth.expert_mx(wl, e, 13)
            np_w["w2"][e], np_w["w2_scale"][e] = synth.expert_mx(wl, e, 2)
    t0 = time.perf_counter()
    OL.moe_layer(xb, logits, bias, np_w, E=wl.E, n_shared=wl.n_shared, n_group=wl.n_group,
                 topk_group=wl.topk_group, topk=wl.topk, afmt=afmt, wfmt=wfmt)
    secs = time.perf_counter() - t0
    return secs, xb.shape[0] * (wl.topk + wl.n_shared), len(experts)


# fixed seeded token subsets of the large workloads for the oracle timing
CPU_SAMPLE_TOKENS = 2


def cpu_baseline(w, args):
    """The oracle as it stands, timed on the host on bounded samples.

    The headline entry is one full step of the T=8 decode workload.  The
    per-config entries: the tiny layer in full; the prefill, skewed-prefill
    and NVFP4 layers on a fixed seeded subset of CPU_SAMPLE_TOKENS tokens of
    their batches (TFLOP/s extrapolated per token: the oracle's time is mostly
    the per-expert weight decode, so the rate grows with the subset); the
    MXFP4 -> FP8 conversion on one expert's gate/up rows (GB/s)."""
    import synth
    from oracle import convert as OC
    cores = len(os.sched_getaffinity(0))
    threads = blas_threads()
    T = 8
    secs, _, n_exp = _oracle_layer_timed(w, T, 1000, "bf16", "mx")
    nbytes = n_exp * (BYTES_W13 + BYTES_W2) + 2 * T * w.H * 2 + T * w.E * 4
    head = dict(value=nbytes / secs / 1e9, unit="GB/s", cores=cores, blas_threads=threads,
                kind="oracle",
                sample=(f"decode layer, one step of {T} tokens ({n_exp} experts, "
                        f"{nbytes/1e6:.1f} MB of weights), NumPy float64 oracle, {secs:.2f} s; "
                        "weight generation excluded"))
    per = {}
    tw = synth.WORKLOADS["tiny"]
    secs, pairs, _ = _oracle_layer_timed(tw, tw.T, 0, "bf16", "mx")
    fl = pairs * (2 * tw.H * 2 * tw.I + 2 * tw.I * tw.H)
    per["tiny"] = dict(value=fl / secs / 1e12, unit="TFLOP/s", seconds=round(secs, 3),
                       sample=f"tiny layer in full (T={tw.T})")
    for key, wname, seed, afmt, wfmt in (("prefill", "prefill", 2000, "mx", "mx"),
                                         ("skewed_prefill", "skewed", 5000, "mx", "mx"),
                                         ("nvfp4", "nvfp4", 4000, "nvfp4", "nvfp4")):
        wl = synth.WORKLOADS[wname]
        toks = np.sort(synth.rng(wl.wid, 90).choice(wl.T, CPU_SAMPLE_TOKENS, replace=False))
        secs, pairs, n_exp = _oracle_layer_timed(wl, wl.T, seed, afmt, wfmt, tokens=toks)
        per[key] = dict(value=FLOP_PER_PAIR * pairs / secs / 1e12, unit="TFLOP/s",
                        seconds=round(secs, 2),
                        sample=(f"tokens {toks.tolist()} of the T={wl.T} batch ({pairs} pairs, "
                                f"{n_exp} experts), extrapolated per token"
                                + ("; the NVFP4 tensor scales span the sample only"
                                   if afmt == "nvfp4" else "")))
        log(args, f"cpu baseline {key}: {per[key]['value']:.2e} TFLOP/s in {secs:.1f} s")
    sw = synth.WORKLOADS["skewed"]
    codes, _ = synth.expert_mx(sw, 0, 13)
    scales, _ = synth.spanned_scales(codes.shape[0], codes.shape[1] // 16, 5, 0)
    t0 = time.perf_counter()
    OC.mxfp4_to_fp8_channel(codes, scales)
    secs = time.perf_counter() - t0
    nbytes = codes.size + scales.size + codes.size * 2 + 5 * codes.shape[0]
    per["fp8_convert"] = dict(value=nbytes / secs / 1e9, unit="GB/s", seconds=round(secs, 2),
                              sample=f"one expert's gate/up rows ({codes.shape[0]} x "
                                     f"{codes.shape[1] * 2})")
    head["per_config"] = per
    return head


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer's "
              "sharding over several GPUs exists only as a design.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import block_scaled_fp4_moe_amd as fm
    import synth
    fm.load()
    if args.copy_calibration:
        # a plain copy kernel of known size: 1 GiB read + 1 GiB written
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = synth.WORKLOADS["decode"]
    t0 = time.time()
    dev_w = make_weights(w, torch)
    torch.cuda.synchronize()
    log(args, f"weights for {w.E + w.n_shared} experts ready in {time.time() - t0:.1f} s")

    head = run_decode(fm, w, dev_w, args.tokens, args.steps, args.warmup, torch, args)
    sweep = {}
    if not args.no_sweep:
        for T in (1, 64):
            if T != args.tokens:
                r = run_decode(fm, w, dev_w, T, args.steps, args.warmup, torch, args)
                sweep[f"T{T}"] = dict(gbs=round(r["gbs"], 1), ms_per_step=round(r["ms_per_step"], 4),
                                      experts_per_step=round(r["touched_per_step"], 1),
                                      frac=round(r["gbs"] / HBM_PEAK_GBS, 4),
                                      step_spread=r["spread"])
    single = {}
    if not args.no_sweep:
        # the same decode batches through the single-launch layer
        # (moe_decode_fused), for comparison with the chain of calls
        for T in (args.tokens, 1):
            if T > 16:
                continue
            r = run_decode(fm, w, dev_w, T, args.steps, args.warmup, torch, args, fused=True)
            single[f"T{T}"] = dict(gbs=round(r["gbs"], 1), us_per_step=round(r["ms_per_step"] * 1e3, 2),
                                  frac=round(r["gbs"] / HBM_PEAK_GBS, 4),
                                  kernels_us={k2: round(v * 1e3, 2)
                                              for k2, v in r["per_kernel_ms"].items()})
    ep = None
    scaling = None
    if not args.no_sweep:
        ep = run_ep_share(fm, w, dev_w, args.tokens, args.steps, args.warmup, torch, args)
        scaling = run_expert_scaling(fm, w, dev_w, torch, args)
    prefill = None
    if not args.no_prefill:
        r = run_prefill(fm, dev_w, args.prefill_steps, torch, args)
        prefill = dict(tflops=round(r["tflops"], 1), ms_per_step=round(r["ms_per_step"], 3),
                       frac=round(r["tflops"] / MXFP4_PEAK_TFLOPS, 4),
                       kernels_ms={k: round(v, 4) for k, v in r["per_kernel_ms"].items()},
                       workload="prefill MoE layer, T=8192, uniform routing, MXFP4 activations "
                                "(mxfp4_quant_1x32) x MXFP4 weights, gfx950 scaled MFMA")
    skewed = None
    if not args.no_prefill:
        skewed = run_skewed_mx(fm, dev_w, args.prefill_steps, torch, args)
    extra = {}
    if not args.no_extra:
        del dev_w
        torch.cuda.empty_cache()
        runs = {"nvfp4": (run_nvfp4, 10), "fp8": (run_fp8, 3), "dense": (run_dense, 10)}
        for name in args.extra:
            fn, steps = runs[name]
            extra[name] = fn(fm, steps, torch, args)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args)
        log(args, f"cpu baseline: {cpu['value']:.3f} GB/s ({cpu['sample']})")

    s1 = head["roofline_kernel"]
    rk_desc = {"fused": "moe_decode_fused (the whole layer in one launch)",
               "stage1": "fp4_grouped_gemm stage 1 (gate/up + SiLU*up), dq path"}[s1["name"]]
    traffic = roofline_traffic(s1["name"], args.tokens)
    line = {
        "metric": METRIC,
        "value": round(head["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"decode MoE layer, T={args.tokens}, hidden 7168, expert intermediate "
                         "2048, 384 routed experts top-8 (8 groups, keep 4) + 1 shared, MXFP4 "
                         "weights decoded to bf16 in-tile, bf16 activations"),
            "tokens": args.tokens,
            "experts_touched_per_step": round(head["touched_per_step"], 2),
            "bytes_per_step": int(head["bytes_per_step"]),
            "routing_draws_rotated": N_ROTATE,
            "weight_layout": "fragment-major (fp4_weight_preshuffle, once at load)",
        },
        "roofline": {
            "kernel": rk_desc,
            "bound": "hbm",
            "achieved": round(s1["gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(s1["gbs"] / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_source": ("stored, not measured by this run: two rocprofv3 --pmc passes "
                               "(FETCH_SIZE, WRITE_SIZE) of this kernel on this workload, "
                               "profiles/dq_gemm_decode_T8_hbm_counters.md; reported only while "
                               "the kernel's sources hash as they did then" if traffic is not None else
                               "null: no counter passes of this kernel as it is now"),
            "avg_launch_us": round(s1["ms"] * 1e3, 2),
            "algorithmic_bytes_per_launch": int(s1["bytes"]),
        },
        "layer_frac_of_hbm_peak": round(head["gbs"] / HBM_PEAK_GBS, 4),
        "kernels_us": {k: round(v * 1e3, 2) for k, v in head["per_kernel_ms"].items()},
        "step_spread": head["spread"],
        "decode_sweep": sweep,
        "decode_single_launch": single,
        "ep_share": ep,
        "decode_expert_scaling": scaling,
        "prefill": prefill,
        "skewed_prefill": skewed,
        "nvfp4": extra.get("nvfp4"),
        "fp8": extra.get("fp8"),
        "dense_linear": extra.get("dense"),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
