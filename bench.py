#!/usr/bin/env python3
"""Benchmark of the fused MoE expert-FFN forward on one MI355X.

One step = the whole hot path on one batch: router (top-k softmax) and the
fused forward (align, gemm1 + SiLU*up, gemm2, combine) for the
Qwen3-235B-shaped bf16 layer (H=4096, I=1536, E=128, top-8) at T=512 tokens,
gate/up passed as views into the packed w13. Inputs are seeded synthetic
tensors already resident in HBM. The JSON line also carries:

* the same layer at T=4096 and T=16384 with router-replay id slices and
  packed views (the other token counts the metric names), bit-checked
  against contiguous copies;
* the pages' layout microbenchmark: contiguous weights against strided
  packed views at 512/4096/16384 tokens, same weights, routes and
  configuration, alternating order (Liger-Kernel PR #1377, Testing Done);
* Zipf-skewed routing with an activation stored transposed, T = 1, 7, 333,
  4099, against a contiguous activation;
* the Qwen3.5-397B TP2-shaped MXFP4 shard per token bucket 1 ... 32768, for
  both routing conventions (512/10 and 513/11);
* the roofline of the dominant kernel (gemm1) with HIP events on its stream
  and the HBM traffic from the committed rocprofv3 counters; the oracle
  timed on the host cores.

Cold timing: before each timed call a 512 MiB write, then a read of it,
evicts the L2 and the 256 MB MALL (the read leaves clean lines, so the call
does not pay for writing back the flush's dirty ones), and HIP events
bracket the call alone (one call captured in a HIP graph and replayed, so
host marshalling is not timed). Warm timing
replays it back to back. Fractions of the roofline use the binding bound:
max(algorithmic bytes / 8 TB/s, flops / MFMA peak) over the measured time;
algorithmic bytes = touched experts' weights (+ scales) + x in + out + ids
and weights. The "pipeline" fraction adds the implementation's own h and y
round trips (written by one kernel, read by the next).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense MXFP4 MFMA
METRIC = "fused-MoE fwd µs/call + TFLOP/s & %roofline at T=512/4096/16384 tokens"
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "gemm1_bf16_qwen3_235b_t512_counters.md")
KERNEL_SOURCES = ("mixture_experts_ffn_align_amd/csrc/gemm_stream.hip",
                  "mixture_experts_ffn_align_amd/csrc/gemm_tile.hip",
                  "mixture_experts_ffn_align_amd/csrc/moe_internal.h")
KERNEL_FAMILY = {1: "gemm_stream", 3: "gemm_tile", 7: "gemm1 per slot", 11: "gemm_stream", 13: "gemm_tile",
                 17: "gemm1 per slot"}
FLUSH_BYTES = 512 << 20
# The pages' tuned MI355X latencies of the 512/10 MXFP4 TP2 shard (aiter PR,
# tuned latency table), quoted as context.
PAGES_MXFP4_US = {1: 25.0, 2: 27.5, 4: 37.2, 8: 54.5, 16: 91.5, 32: 140.8, 64: 204.1, 128: 253.0, 256: 278.2,
                  512: 288.0, 1024: 306.9, 2048: 378.7, 4096: 557.9, 8192: 859.0, 16384: 1507.1, 32768: 2770.5}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float(0)
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


class Timer:
    """Warm and cold GPU time of one call captured in a HIP graph."""

    def __init__(self, dev):
        import torch
        self.torch = torch
        self.hip = HipEvents()
        self.flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        self.ev = self.hip.create(2)

    def stream(self):
        return self.torch.cuda.current_stream().cuda_stream

    def graph(self, call):
        """Capture call() (which returns its output tensor) after eager runs
        on a side stream; the replay must reproduce the eager bits."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(2):
                out = call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        eager = out.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            out = call()
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, eager):
            raise RuntimeError("graph replay differs from the eager call")
        return g

    def cold(self, g, n):
        """Per-call µs (median, p10, p90) with L2 and MALL flushed first: a
        512 MiB write, then a read of the same buffer, so the caches hold
        clean lines of the flush buffer and the timed call neither hits on
        its own data nor pays for writing back the flush's dirty lines."""
        s = self.stream()
        ts = []
        for _ in range(n):
            self.flush.fill_(1.0)
            self.flush_sum = self.flush.amax()
            self.hip.record(self.ev[0], s)
            g.replay()
            self.hip.record(self.ev[1], s)
            self.torch.cuda.synchronize()
            ts.append(self.hip.elapsed_ms(self.ev[0], self.ev[1]) * 1e3)
        ts.sort()
        return ts[len(ts) // 2], ts[len(ts) // 10], ts[(9 * len(ts)) // 10]

    def warm(self, g, reps):
        s = self.stream()
        g.replay()
        self.hip.record(self.ev[0], s)
        for _ in range(reps):
            g.replay()
        self.hip.record(self.ev[1], s)
        self.torch.cuda.synchronize()
        return self.hip.elapsed_ms(self.ev[0], self.ev[1]) * 1e3 / reps

    def both(self, call, n_cold=10, reps=None):
        g = self.graph(call)
        cold = self.cold(g, n_cold)
        warm = self.warm(g, reps or max(3, min(200, int(2e5 / (cold[0] + 20)))))
        del g
        return cold, warm


def source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per gemm1 launch from the committed rocprofv3 counter runs,
    or None when the kernel source changed since they were taken."""
    if not os.path.exists(PROFILE_COUNTERS):
        return None
    text = open(PROFILE_COUNTERS).read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("source_hash") != source_hash():
        return None
    return d.get("traffic_bytes_per_launch")


def fractions(byts, flops, peak_tflops, us, extra_bytes=0):
    """Binding-roofline fraction, the bound, and the pipeline fraction."""
    hbm_s, mfma_s = byts / (HBM_PEAK_GBS * 1e9), flops / (peak_tflops * 1e12)
    pipe_s = (byts + extra_bytes) / (HBM_PEAK_GBS * 1e9)
    return {
        "bound": "hbm" if hbm_s >= mfma_s else "mfma",
        "roofline_frac": round(max(hbm_s, mfma_s) / (us * 1e-6), 3),
        "pipeline_frac": round(max(pipe_s, mfma_s) / (us * 1e-6), 3),
        "tflops": round(flops / (us * 1e-6) / 1e12, 1),
        "hbm_gbs": round(byts / (us * 1e-6) / 1e9, 1),
    }


def hy_bytes(cfg, A, H, I, fp4):
    """The implementation's own intermediate traffic: h written by gemm1 and
    read by gemm2, y written by gemm2 and read by the combine (none when
    gemm2 folds the combine in)."""
    hb = (I // 2 + I // 32) if fp4 else 2 * I
    fused = cfg["gemm2_kernel"] in (6, 16)
    return 2 * A * hb + (0 if fused else 2 * A * H * 2)


def cfg_brief(cfg):
    return {kk: cfg[kk] for kk in ("config_index", "block_m", "block_m2", "gemm1_kernel", "gemm2_kernel",
                                   "gemm1_split_k", "gemm2_split_k")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget for the oracle's CPU baseline sample (0 to skip)")
    ap.add_argument("--no-extra", action="store_true",
                    help="only the headline step: skip the other token counts, layouts and MXFP4 buckets")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy three times (counter calibration)")
    ap.add_argument("--mxfp4", default="",
                    help="comma-separated token buckets: instead of the bf16 line, one JSON line per "
                         "bucket for the MXFP4 TP2 shard")
    ap.add_argument("--routing", default="512", choices=["512", "513"],
                    help="with --mxfp4: 512 experts top-10, or 513 with the shared expert (top-11)")
    ap.add_argument("--bf16", default="",
                    help="comma-separated token buckets: one JSON line per bucket for the bf16 "
                         "Qwen3-235B-shaped layer (fused forward on router ids, packed w13 views)")
    ap.add_argument("--ep", type=int, default=0,
                    help="with --bf16: time one expert-parallel shard of S (experts [0, E/S), global "
                         "ids, per-slot rows out) and the tokens' home combine instead of the whole layer")
    ap.add_argument("--norm", default="",
                    help="comma-separated token counts: the RMSNorm pre-pass on its own (contiguous and "
                         "transposed x) and inside the bf16 fused forward, one JSON line each")
    ap.add_argument("--bwd", default="",
                    help="comma-separated token counts: the backward of the bf16 Qwen3-235B-shaped layer "
                         "(fp32 weight gradients), one JSON line each")
    ap.add_argument("--config", type=int, default=-1,
                    help="with --mxfp4/--bf16: force this tile-config index (comparisons; -1 = the built-in choice)")
    ap.add_argument("--calls", type=int, default=0,
                    help="with --mxfp4/--bf16: only this many eager calls per bucket, no timing "
                         "(a short run for counter passes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(multi-GPU expert/tensor parallel sharding is a design note, not built).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        src = torch.ones(2 ** 28, dtype=torch.float32, device=dev)     # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copied 1 GiB three times")
        return
    if args.mxfp4:
        for line in mxfp4_lines([int(t) for t in args.mxfp4.split(",")], args.routing, dev, args.calls,
                                force=args.config):
            print(json.dumps(line), flush=True)
        return
    if args.norm:
        norm_lines([int(t) for t in args.norm.split(",")], dev)
        return
    if args.bwd:
        bwd_lines([int(t) for t in args.bwd.split(",")], dev)
        return
    if args.bf16 and args.ep > 1:
        ep_buckets([int(t) for t in args.bf16.split(",")], args.ep, dev)
        return
    if args.bf16:
        for line in bf16_lines([int(t) for t in args.bf16.split(",")], dev, args.calls, force=args.config):
            print(json.dumps(line), flush=True)
        return
    headline(args, dev)


def headline(args, dev):
    import numpy as np
    import torch
    import mixture_experts_ffn_align_amd as moe
    from mixture_experts_ffn_align_amd import workloads as W

    sh = W.QWEN3_235B_BF16
    T, H, I, E, k = 512, sh.hidden, sh.inter, sh.experts, sh.top_k
    log(f"[bench] drawing weights {sh.name}")
    g = torch.Generator(device=dev).manual_seed(0)
    w13, w2 = W.draw_weights(sh, g, dev)
    inp = W.make_inputs(sh, T, seed=0, device=dev, weights=(w13, w2))
    gate, up = W.packed_views(w13, I)
    x, logits = inp["x"], inp["logits"]
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    wts = torch.empty(T, k, dtype=torch.float32, device=dev)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(moe.moe_fused_workspace_size(x, gate, up, w2, ids, wts), dtype=torch.uint8,
                     device=dev)
    cfg = moe.moe_query_config(x, gate, up, w2, ids, wts)
    stream = torch.cuda.current_stream().cuda_stream
    hip = HipEvents()
    nst = len(moe.STAGES)

    def step(evs=None):
        if evs is not None:
            hip.record(evs[0], stream)
        moe.moe_topk_softmax(logits, k, ids=ids, weights=wts, stream=stream)
        if evs is not None:
            hip.record(evs[1], stream)
        moe.moe_fused_fwd(x, gate, up, w2, ids, wts, out=out, workspace=ws,
                          stage_events=None if evs is None else evs[2:], stream=stream)
        return out

    def step_g1(ev2):
        """One step with only gemm1 bracketed by events (the roofline's kernel)."""
        moe.moe_topk_softmax(logits, k, ids=ids, weights=wts, stream=stream)
        evs = [0] * (2 * nst)
        evs[2 * 2], evs[2 * 2 + 1] = ev2
        moe.moe_fused_fwd(x, gate, up, w2, ids, wts, out=out, workspace=ws, stage_events=evs, stream=stream)

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: K steps, events only around gemm1 (every stage bracketed
    # would add ~2 us of markers per event to the steps being timed)
    g1sets = [hip.create(2) for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step_g1(g1sets[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    g1_live_ms = sum(hip.elapsed_ms(a, b) for a, b in g1sets) / args.steps
    for evs in g1sets:
        hip.destroy(evs)
    # per-stage breakdown: a separate, untimed pass with every stage bracketed
    evsets = [hip.create(2 + 2 * nst) for _ in range(args.steps)]
    for i in range(args.steps):
        step(evsets[i])
    torch.cuda.synchronize()
    stage_ms = {"route": 0.0}
    stage_ms.update({s: 0.0 for s in moe.STAGES})
    for evs in evsets:
        stage_ms["route"] += hip.elapsed_ms(evs[0], evs[1])
        for s, name in enumerate(moe.STAGES):
            stage_ms[name] += hip.elapsed_ms(evs[2 + 2 * s], evs[3 + 2 * s])
    for key in stage_ms:
        stage_ms[key] /= args.steps
    for evs in evsets:
        hip.destroy(evs)

    touched = int(torch.unique(ids).numel())
    A = T * k
    per_expert = 3 * I * H * 2
    bytes_call = touched * per_expert + 2 * T * H * 2 + 8 * A + T * sh.routed_experts * 4
    flops_call = 6 * H * I * A
    us = ms_per_step * 1e3
    g1_bytes = touched * 2 * I * H * 2 + T * H * 2
    g1_gbs = g1_bytes / (g1_live_ms * 1e-3) / 1e9
    traffic = read_traffic()

    timer = Timer(dev)

    def step_current_stream():
        moe.moe_topk_softmax(logits, k, ids=ids, weights=wts)
        return moe.moe_fused_fwd(x, gate, up, w2, ids, wts, out=out, workspace=ws)
    (cold_us, cold_p10, cold_p90), warm_us = timer.both(step_current_stream, n_cold=15)

    extra = {}
    if not args.no_extra:
        extra = extra_lines(sh, w13, w2, gate, up, dev, timer)

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(inp, w13, w2, T, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(us, 2),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "Qwen3-235B-shaped MoE layer, bf16, T=512 tokens, H=4096, I=1536, E=128, top-8, "
                        "router + fused forward, gate/up as packed w13 views",
            "tokens": T, "hidden": H, "inter": I, "experts": E, "top_k": k,
            "block_m": cfg["block_m"], "gemm1_split_k": cfg["gemm1_split_k"],
        },
        "touched_experts": touched,
        "algorithmic_bytes_per_call": bytes_call,
        **fractions(bytes_call, flops_call, BF16_PEAK_TFLOPS, us, hy_bytes(cfg, A, H, I, False)),
        "cold_us_per_call": {"median": round(cold_us, 1), "p10": round(cold_p10, 1), "p90": round(cold_p90, 1),
                             "how": "512 MiB write then read before each call (L2 and MALL evicted, left clean), "
                                    "events around the graph-replayed step (router + fused forward)"},
        "cold_roofline_frac": round(max(bytes_call / (HBM_PEAK_GBS * 1e9),
                                        flops_call / (BF16_PEAK_TFLOPS * 1e12)) / (cold_us * 1e-6), 3),
        "warm_graph_us_per_call": round(warm_us, 1),
        "stage_us": {kk: round(v * 1e3, 1) for kk, v in stage_ms.items()},
        "gemm1_us_timed_region": round(g1_live_ms * 1e3, 1),
        "roofline": {
            "kernel": f"gemm1 ({KERNEL_FAMILY.get(cfg['gemm1_kernel'], '?')} bf16 stage 1, "
                      f"block_m={cfg['block_m']})",
            "bound": "hbm",
            "achieved": round(g1_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(g1_gbs / HBM_PEAK_GBS, 3),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": g1_bytes,
        },
        **extra,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def extra_lines(sh, w13, w2, gate, up, dev, timer):
    """The other token counts, the layout microbenchmark, the Zipf/transposed
    workload and the MXFP4 buckets (each cold- and warm-timed)."""
    import torch
    import mixture_experts_ffn_align_amd as moe
    from mixture_experts_ffn_align_amd import workloads as W

    H, I, E, k = sh.hidden, sh.inter, sh.experts, sh.top_k
    per_expert = 3 * I * H * 2
    hip = timer.hip
    nst = len(moe.STAGES)
    stream = timer.stream()
    res = {"per_tokens": {}, "layout_microbench": {}, "zipf_transposed_x": {}}
    gc, uc = gate.contiguous(), up.contiguous()
    for TT in (4096, 16384):
        log(f"[bench] T={TT} router-replay slices, packed views")
        ri = W.make_inputs(sh, TT, seed=0, device=dev, routing="replay", weights=(w13, w2))
        x, ids_s, w_s = ri["x"], ri["topk_ids"], ri["topk_weights"]
        ids_c, w_c = ids_s.contiguous(), w_s.contiguous()
        outs = {v: torch.empty(TT, H, dtype=torch.bfloat16, device=dev) for v in ("s", "c")}
        wsx = torch.empty(moe.moe_fused_workspace_size(x, gate, up, w2, ids_s, w_s), dtype=torch.uint8, device=dev)
        strided = lambda: moe.moe_fused_fwd(x, gate, up, w2, ids_s, w_s, out=outs["s"], workspace=wsx)
        contig = lambda: moe.moe_fused_fwd(x, gc, uc, w2, ids_c, w_c, out=outs["c"], workspace=wsx)
        (cs, _, _), warm = timer.both(strided, n_cold=8)
        # stage split from eager calls with events
        ev = hip.create(2 + 2 * nst)
        g1 = g2 = 0.0
        for _ in range(3):
            moe.moe_fused_fwd(x, gate, up, w2, ids_s, w_s, out=outs["s"], workspace=wsx, stage_events=ev[2:],
                              stream=stream)
            torch.cuda.synchronize()
            g1 += hip.elapsed_ms(ev[2 + 2 * 2], ev[3 + 2 * 2]) / 3
            g2 += hip.elapsed_ms(ev[2 + 2 * 3], ev[3 + 2 * 3]) / 3
        hip.destroy(ev)
        cfg = moe.moe_query_config(x, gate, up, w2, ids_s, w_s)
        A = TT * k
        touched = int(torch.unique(ids_s).numel())
        byts = touched * per_expert + 2 * TT * H * 2 + 8 * A
        flops = 6 * H * I * A
        res["per_tokens"][str(TT)] = {
            "us_per_call": round(cs, 1), "timing": "cold (L2 and MALL flushed), graph-replayed fused forward",
            "warm_us_per_call": round(warm, 1),
            **fractions(byts, flops, BF16_PEAK_TFLOPS, cs, hy_bytes(cfg, A, H, I, False)),
            "gemm1_us": round(g1 * 1e3, 1), "gemm2_us": round(g2 * 1e3, 1),
            "gemm1_mfma_frac": round(4 * H * I * A / (g1 * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 3),
            "gemm2_mfma_frac": round(2 * H * I * A / (g2 * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 3),
            "config": cfg_brief(cfg),
            "inputs": "packed w13 views, ids/weights [:, :, 7, :] of [1,T,46,8] (token stride 368)",
        }
        res["layout_microbench"][str(TT)] = layout_pair(timer, strided, contig, outs)
        del ri, x, ids_s, w_s, ids_c, w_c, outs, wsx
        torch.cuda.empty_cache()
    # layout microbenchmark at 512 tokens as well (the pages' first row)
    ri = W.make_inputs(sh, 512, seed=0, device=dev, routing="replay", weights=(w13, w2))
    x, ids_s, w_s = ri["x"], ri["topk_ids"], ri["topk_weights"]
    ids_c, w_c = ids_s.contiguous(), w_s.contiguous()
    outs = {v: torch.empty(512, H, dtype=torch.bfloat16, device=dev) for v in ("s", "c")}
    wsx = torch.empty(moe.moe_fused_workspace_size(x, gate, up, w2, ids_s, w_s), dtype=torch.uint8, device=dev)
    res["layout_microbench"]["512"] = layout_pair(
        timer, lambda: moe.moe_fused_fwd(x, gate, up, w2, ids_s, w_s, out=outs["s"], workspace=wsx),
        lambda: moe.moe_fused_fwd(x, gc, uc, w2, ids_c, w_c, out=outs["c"], workspace=wsx), outs)
    res["layout_microbench"] = {"what": "contiguous gate/up/ids/weights vs packed w13 views and replay slices; "
                                        "same weights, routes and configuration; cold calls in alternating "
                                        "order (Liger-Kernel PR #1377, Testing Done); outputs bit-identical",
                                **{t: res["layout_microbench"][t] for t in ("512", "4096", "16384")}}
    del gc, uc, ri, x, ids_s, w_s, ids_c, w_c, outs, wsx
    torch.cuda.empty_cache()
    # Zipf-skewed routing, transposed activation
    for TT in (1, 7, 333, 4099):
        zi = W.make_inputs(sh, TT, seed=0, device=dev, logits_kind="zipf", x_layout="transposed",
                           weights=(w13, w2))
        ids, wts = moe.moe_topk_softmax(zi["logits"], k)
        xt, xc = zi["x"], zi["x"].contiguous()
        outs = {v: torch.empty(TT, H, dtype=torch.bfloat16, device=dev) for v in ("s", "c")}
        wsx = torch.empty(moe.moe_fused_workspace_size(xt, gate, up, w2, ids, wts), dtype=torch.uint8, device=dev)
        pair = layout_pair(timer, lambda: moe.moe_fused_fwd(xt, gate, up, w2, ids, wts, out=outs["s"], workspace=wsx),
                           lambda: moe.moe_fused_fwd(xc, gate, up, w2, ids, wts, out=outs["c"], workspace=wsx),
                           outs, keys=("transposed_x_us", "contiguous_x_us"))
        touched = int(torch.unique(ids).numel())
        A = TT * k
        byts = touched * per_expert + 2 * TT * H * 2 + 8 * A
        cfg = moe.moe_query_config(xt, gate, up, w2, ids, wts)
        res["zipf_transposed_x"][str(TT)] = {
            **pair, "touched_experts": touched,
            **fractions(byts, 6 * H * I * A, BF16_PEAK_TFLOPS, pair["transposed_x_us"], hy_bytes(cfg, A, H, I, False)),
            "config": cfg_brief(cfg)}
        del zi, ids, wts, xt, xc, outs, wsx
        torch.cuda.empty_cache()
    res["zipf_transposed_x"] = {"what": "router on Zipf(1.2)-skewed logits (4 experts never chosen), x stored "
                                        "transposed [4096, T] and passed as [T, 4096] with stride (1, T); "
                                        "fused forward cold-timed against a contiguous copy of x",
                                **res["zipf_transposed_x"]}
    # MXFP4 TP2 shard, both routings
    res["mxfp4_tp2"] = {}
    for routing in ("512", "513"):
        lines = mxfp4_lines([1 << i for i in range(16)], routing, dev, 0, timer=timer)
        res["mxfp4_tp2"][routing] = {str(l["tokens"]): {kk: l[kk] for kk in (
            "us_per_call", "warm_us_per_call", "touched_experts", "bound", "roofline_frac", "pipeline_frac",
            "tflops", "hbm_gbs", "pages_tuned_us") if kk in l} | {"config": l["config"]["config_index"]}
            for l in lines}
    res["mxfp4_tp2"]["what"] = ("Qwen3.5-397B TP2-shaped MXFP4 shard (H=4096, I=512), fused forward on router "
                                "ids, cold-timed; 512 = 512 experts top-10, 513 = shared expert 512 appended "
                                "(top-11); pages_tuned_us = the pages' tuned 512/10 latency, context only")
    return res


def layout_pair(timer, a, b, outs, keys=("strided_us", "contiguous_us"), rounds=6):
    """Cold per-call times of two variants run in alternating order; their
    outputs must be bit-identical."""
    import torch
    ga, gb = timer.graph(a), timer.graph(b)
    if not torch.equal(outs["s"], outs["c"]):
        raise RuntimeError("layout variants differ")
    ta, tb = [], []
    for r in range(rounds):
        first, second = (ga, gb) if r % 2 == 0 else (gb, ga)
        t1 = timer.cold(first, 1)[0]
        t2 = timer.cold(second, 1)[0]
        if first is ga:
            ta.append(t1)
            tb.append(t2)
        else:
            tb.append(t1)
            ta.append(t2)
    ta.sort()
    tb.sort()
    ma, mb = ta[len(ta) // 2], tb[len(tb) // 2]
    del ga, gb
    return {keys[0]: round(ma, 1), keys[1]: round(mb, 1), "difference_pct": round(100.0 * (ma - mb) / mb, 2),
            "bit_identical": True}


def bf16_lines(buckets, dev, calls=0, force=-1):
    """bf16 Qwen3-235B-shaped layer: per token bucket, the fused forward on
    router ids computed beforehand, gate/up as packed w13 views."""
    import torch
    import mixture_experts_ffn_align_amd as moe
    from mixture_experts_ffn_align_amd import workloads as W

    sh = W.QWEN3_235B_BF16
    H, I, E, k = sh.hidden, sh.inter, sh.experts, sh.top_k
    log(f"[bench] drawing weights {sh.name}")
    g = torch.Generator(device=dev).manual_seed(0)
    w13, w2 = W.draw_weights(sh, g, dev)
    gate, up = W.packed_views(w13, I)
    per_expert = 3 * I * H * 2
    timer = Timer(dev) if not calls else None
    lines = []
    for T in buckets:
        inp = W.make_inputs(sh, T, seed=T, device=dev, weights=(w13, w2))
        ids, wts = moe.moe_topk_softmax(inp["logits"], k)
        out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        fk = dict(force_config=force)
        ws = torch.empty(moe.moe_fused_workspace_size(inp["x"], gate, up, w2, ids, wts, **fk), dtype=torch.uint8,
                         device=dev)
        cfg = moe.moe_query_config(inp["x"], gate, up, w2, ids, wts, **fk)
        call = lambda: moe.moe_fused_fwd(inp["x"], gate, up, w2, ids, wts, out=out, workspace=ws, **fk)
        if calls:
            for _ in range(calls):
                call()
            torch.cuda.synchronize()
            continue
        (cold, p10, p90), warm = timer.both(call, n_cold=10)
        touched = int(torch.unique(ids).numel())
        A = T * k
        byts = touched * per_expert + T * H * 2 * 2 + 8 * A
        line = {
            "workload": f"{sh.name}, fused forward on given top-k ids/weights, packed w13 views",
            "tokens": T, "touched_experts": touched, "us_per_call": round(cold, 1),
            "us_p10_p90": [round(p10, 1), round(p90, 1)], "warm_us_per_call": round(warm, 1),
            "timing": "cold: L2 and MALL flushed (512 MiB write, then read) before each graph-replayed call; warm: replays back to back",
            "algorithmic_bytes": byts,
            **fractions(byts, 6 * H * I * A, BF16_PEAK_TFLOPS, cold, hy_bytes(cfg, A, H, I, False)),
            "config": cfg_brief(cfg),
        }
        lines.append(line)
        log(f"[bench] bf16 T={T}: {cold:.1f} us cold, {warm:.1f} us warm")
        del inp, ids, wts, out, ws
        torch.cuda.empty_cache()
    return lines


def mxfp4_lines(buckets, routing, dev, calls=0, timer=None, force=-1):
    """MXFP4 TP2 shard (H=4096, I=512; 512 experts top-10, or 513 with the
    shared expert): per token bucket, the fused forward (align + activation
    quantisation, gemm1 + SiLU*up with h quantised, gemm2, combine) on router
    ids/weights computed beforehand."""
    import torch
    import mixture_experts_ffn_align_amd as moe
    from mixture_experts_ffn_align_amd import workloads as W

    sh = W.QWEN35_397B_TP2_FP4_512 if routing == "512" else W.QWEN35_397B_TP2_FP4_513
    H, I, E, k = sh.hidden, sh.inter, sh.experts, sh.top_k
    log(f"[bench] drawing and quantising weights {sh.name}")
    g = torch.Generator(device=dev).manual_seed(0)
    w13, w2 = W.draw_weights(sh, g, dev)
    gate, up = W.packed_views(w13, I)
    (gq, gs), (uq, us), (wq, wsc) = moe.moe_quant_mxfp4(gate), moe.moe_quant_mxfp4(up), moe.moe_quant_mxfp4(w2)
    del w13, w2, gate, up
    torch.cuda.empty_cache()
    if timer is None and not calls:
        timer = Timer(dev)
    hip = HipEvents()
    nst = len(moe.STAGES)
    per_expert = 3 * I * H // 2 + 3 * I * H // 32          # e2m1 codes + e8m0 scales of gate, up, down
    lines = []
    for T in buckets:
        gx = torch.Generator(device=dev).manual_seed(T)
        x = torch.randn(T, H, generator=gx, device=dev).to(torch.bfloat16)
        logits = torch.randn(T, sh.routed_experts, generator=gx, device=dev)
        ids, wts = moe.moe_topk_softmax(logits, sh.routed_k, shared_id=sh.shared_expert, shared_w=1.0)
        out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        kw = dict(gate_scale=gs, up_scale=us, w2_scale=wsc, mode=moe.MODE_MXFP4, force_config=force)
        ws = torch.empty(moe.moe_fused_workspace_size(x, gq, uq, wq, ids, wts, **kw), dtype=torch.uint8, device=dev)
        cfg = moe.moe_query_config(x, gq, uq, wq, ids, wts, **kw)
        call = lambda: moe.moe_fused_fwd(x, gq, uq, wq, ids, wts, out=out, workspace=ws, **kw)
        if calls:
            for _ in range(calls):
                call()
            torch.cuda.synchronize()
            log(f"[bench] mxfp4 {routing} T={T}: {calls} calls")
            continue
        (cold, p10, p90), warm = timer.both(call, n_cold=10)
        stream = torch.cuda.current_stream().cuda_stream
        evs = hip.create(2 * nst)
        st = {s: [] for s in moe.STAGES}
        for _ in range(5):
            moe.moe_fused_fwd(x, gq, uq, wq, ids, wts, out=out, workspace=ws, stage_events=evs, stream=stream, **kw)
            torch.cuda.synchronize()
            for i, s in enumerate(moe.STAGES):
                st[s].append(hip.elapsed_ms(evs[2 * i], evs[2 * i + 1]) * 1e3)
        hip.destroy(evs)
        touched = int(torch.unique(ids).numel())
        A = T * k
        byts = touched * per_expert + T * H * 2 * 2 + 8 * A
        line = {
            "workload": f"{sh.name}, fused forward on given top-k ids/weights",
            "tokens": T, "touched_experts": touched, "us_per_call": round(cold, 1),
            "us_p10_p90": [round(p10, 1), round(p90, 1)], "warm_us_per_call": round(warm, 1),
            "timing": "cold: L2 and MALL flushed (512 MiB write, then read) before each graph-replayed call; warm: replays back to back",
            "algorithmic_bytes": byts,
            **fractions(byts, 6 * H * I * A, FP4_PEAK_TFLOPS, cold, hy_bytes(cfg, A, H, I, True)),
            "stage_us_eager_events": {s: round(sorted(v)[len(v) // 2], 1) for s, v in st.items()},
            "config": cfg_brief(cfg),
        }
        if routing == "512":
            line["pages_tuned_us"] = PAGES_MXFP4_US.get(T)
        lines.append(line)
        log(f"[bench] mxfp4 {routing} T={T}: {cold:.1f} us cold, {warm:.1f} us warm")
        del x, logits, ids, wts, out, ws
        torch.cuda.empty_cache()
    return lines


def ep_buckets(buckets, S, dev):
    """One expert-parallel shard of the bf16 Qwen3-235B-shaped layer: shard 0
    of S holds experts [0, E/S) as views into packed w13, takes the global
    top-8 ids, and writes the per-slot rows of its slots (what an all-to-all
    would return to the tokens' home ranks); then the home combine of all T*k
    rows. Both cold-timed; inputs as in --bf16."""
    import torch
    import mixture_experts_ffn_align_amd as moe
    from mixture_experts_ffn_align_amd import workloads as W

    sh = W.QWEN3_235B_BF16
    H, I, E, k = sh.hidden, sh.inter, sh.experts, sh.top_k
    es = E // S
    log(f"[bench] drawing weights {sh.name}")
    g = torch.Generator(device=dev).manual_seed(0)
    w13, w2 = W.draw_weights(sh, g, dev)
    gate, up = W.packed_views(w13, I)
    gs, us, w2s = gate[:es], up[:es], w2[:es]
    per_expert = 3 * I * H * 2
    timer = Timer(dev)
    for T in buckets:
        inp = W.make_inputs(sh, T, seed=T, device=dev, weights=(w13, w2))
        ids, wts = moe.moe_topk_softmax(inp["logits"], k)
        y = torch.zeros((T, k, H), dtype=torch.bfloat16, device=dev)   # foreign rows stay 0
        out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        kw = dict(expert_offset=0, num_global_experts=E, y_rows=y)
        ws = torch.empty(moe.moe_fused_workspace_size(inp["x"], gs, us, w2s, ids, wts, **kw),
                         dtype=torch.uint8, device=dev)
        (us_shard, _, _), _ = timer.both(lambda: moe.moe_fused_fwd(inp["x"], gs, us, w2s, ids, wts, workspace=ws,
                                                                  **kw))
        (us_comb, _, _), _ = timer.both(lambda: moe.moe_combine(y, ids, wts, E, out=out))
        local = (ids < es)
        n_local = int(local.sum().item())
        touched = int(torch.unique(ids[local]).numel())
        byts = touched * per_expert + T * H * 2 + n_local * H * 2 + 4 * T * k
        flops = 6 * H * I * n_local
        comb_bytes = T * k * H * 2 + T * H * 2 + 8 * T * k
        print(json.dumps({
            "workload": f"{sh.name}, expert-parallel shard 0 of {S} (experts [0, {es})), global ids, "
                        "per-slot rows out; then the home combine of all rows",
            "tokens": T, "local_slots": n_local, "touched_local_experts": touched,
            "shard_us_per_call": round(us_shard, 1),
            "shard_algorithmic_bytes": byts,
            **{"shard_" + kk: v for kk, v in fractions(byts, flops, BF16_PEAK_TFLOPS, us_shard).items()},
            "combine_us_per_call": round(us_comb, 1),
            "combine_hbm_gbs": round(comb_bytes / (us_comb * 1e-6) / 1e9, 1),
            "timing": "cold: L2 and MALL flushed before each graph-replayed call",
        }), flush=True)
        del inp, ids, wts, y, out, ws
        torch.cuda.empty_cache()


def bwd_lines(tokens, dev):
    """Backward of the bf16 Qwen3-235B-shaped layer: gradients of sum(dout * out)
    for x, the top-k weights and all three weight tensors (fp32), one call
    graph-timed cold, with the weight gradients overwritten and with them
    accumulated (added to the given ones, experts without slots untouched).
    Algorithmic flops: 16 H I per slot (recompute 4, q 2, dx 4, dW2 2, dW13
    4); bytes: touched experts' w13 read twice and w2 once in bf16, plus the
    fp32 gradients of all E experts written (overwrite) or of the touched
    experts read and written (accumulate), plus x, dout and dx."""
    import torch
    import mixture_experts_ffn_align_amd as moe
    from mixture_experts_ffn_align_amd import workloads as W

    sh = W.QWEN3_235B_BF16
    H, I, E, k = sh.hidden, sh.inter, sh.experts, sh.top_k
    log(f"[bench] drawing weights {sh.name}")
    g = torch.Generator(device=dev).manual_seed(0)
    w13, w2 = W.draw_weights(sh, g, dev)
    gate, up = W.packed_views(w13, I)
    dgate = torch.empty((E, I, H), dtype=torch.float32, device=dev)
    dup = torch.empty_like(dgate)
    dw2 = torch.empty((E, H, I), dtype=torch.float32, device=dev)
    timer = Timer(dev)
    for T in tokens:
        inp = W.make_inputs(sh, T, seed=T, device=dev, weights=(w13, w2))
        ids, wts = moe.moe_topk_softmax(inp["logits"], k)
        dout = torch.randn(T, H, generator=torch.Generator(device=dev).manual_seed(T + 7), device=dev).to(torch.bfloat16)
        dx = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        dwt = torch.empty(T, k, dtype=torch.float32, device=dev)
        ws = torch.empty(moe.moe_fused_bwd_workspace_size(inp["x"], gate, up, w2, ids, wts, dout),
                         dtype=torch.uint8, device=dev)

        def call(accumulate=False):
            moe.moe_fused_bwd(inp["x"], gate, up, w2, ids, wts, dout, dx=dx, dgate=dgate, dup=dup, dw2=dw2,
                              dtopk_weights=dwt, workspace=ws, accumulate=accumulate)
            return dx
        (us, _, _), _ = timer.both(call, n_cold=5, reps=5)
        (us_acc, _, _), _ = timer.both(lambda: call(True), n_cold=5, reps=5)
        touched = int(torch.unique(ids).numel())
        A = T * k
        flops = 16 * H * I * A
        common = touched * (2 * 2 * I * H * 2 + I * H * 2) + T * H * 2 * 3 + 8 * A
        byts = common + E * 3 * I * H * 4
        byts_acc = common + touched * 3 * I * H * 4 * 2
        mfma_s = flops / (BF16_PEAK_TFLOPS * 1e12)

        def frac(b, t):
            return round(max(b / (HBM_PEAK_GBS * 1e9), mfma_s) / (t * 1e-6), 3)
        print(json.dumps({
            "workload": f"{sh.name} backward: dx, top-k weight, gate/up/w2 gradients (fp32), packed w13 views",
            "tokens": T, "touched_experts": touched, "us_per_call": round(us, 1),
            "tflops": round(flops / (us * 1e-6) / 1e12, 1), "algorithmic_bytes": byts,
            "bound": "hbm" if byts / (HBM_PEAK_GBS * 1e9) >= mfma_s else "mfma",
            "roofline_frac": frac(byts, us),
            "accumulate_us_per_call": round(us_acc, 1), "accumulate_algorithmic_bytes": byts_acc,
            "accumulate_roofline_frac": frac(byts_acc, us_acc),
            "timing": "cold: L2 and MALL flushed before each graph-replayed call",
        }), flush=True)
        del inp, ids, wts, dout, dx, dwt, ws
        torch.cuda.empty_cache()


def norm_lines(tokens, dev):
    """RMSNorm of H=4096 bf16 rows (weight fp32 uniform [0, 1), eps 1e-6):
    moe_rmsnorm on a contiguous and on a transposed x, and the bf16
    Qwen3-235B-shaped fused forward with and without norm_weight, on a
    contiguous and on a transposed x. Cold-timed."""
    import torch
    import mixture_experts_ffn_align_amd as moe
    from mixture_experts_ffn_align_amd import workloads as W

    sh = W.QWEN3_235B_BF16
    H, I, k = sh.hidden, sh.inter, sh.top_k
    log(f"[bench] drawing weights {sh.name}")
    g = torch.Generator(device=dev).manual_seed(0)
    w13, w2 = W.draw_weights(sh, g, dev)
    gate, up = W.packed_views(w13, I)
    nw = torch.rand(H, generator=torch.Generator().manual_seed(1)).to(dev)
    timer = Timer(dev)
    for T in tokens:
        inp = W.make_inputs(sh, T, seed=T, device=dev, weights=(w13, w2))
        x = inp["x"]
        xt = x.t().contiguous().t()
        xn = torch.empty_like(x)
        ids, wts = moe.moe_topk_softmax(inp["logits"], k)
        out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        ws = torch.empty(moe.moe_fused_workspace_size(xt, gate, up, w2, ids, wts, norm_weight=nw),
                         dtype=torch.uint8, device=dev)
        (us_rows, _, _), _ = timer.both(lambda: moe.moe_rmsnorm(x, nw, 1e-6, out=xn))
        (us_cols, _, _), _ = timer.both(lambda: moe.moe_rmsnorm(xt, nw, 1e-6, out=xn))
        (us_f, _, _), _ = timer.both(lambda: moe.moe_fused_fwd(x, gate, up, w2, ids, wts, out=out, workspace=ws))
        (us_fn, _, _), _ = timer.both(lambda: moe.moe_fused_fwd(x, gate, up, w2, ids, wts, out=out, workspace=ws,
                                                                norm_weight=nw, norm_eps=1e-6))
        (us_ft, _, _), _ = timer.both(lambda: moe.moe_fused_fwd(xt, gate, up, w2, ids, wts, out=out, workspace=ws))
        (us_fnt, _, _), _ = timer.both(lambda: moe.moe_fused_fwd(xt, gate, up, w2, ids, wts, out=out, workspace=ws,
                                                                 norm_weight=nw, norm_eps=1e-6))
        byts = T * H * 2 * 2 + H * 4
        print(json.dumps({
            "workload": f"RMSNorm of [T, {H}] bf16 rows, fp32 weight; {sh.name} fused forward with it",
            "tokens": T,
            "rmsnorm_us": round(us_rows, 2), "rmsnorm_gbs": round(byts / (us_rows * 1e-6) / 1e9, 1),
            "rmsnorm_hbm_frac": round(byts / (us_rows * 1e-6) / 1e9 / HBM_PEAK_GBS, 3),
            "rmsnorm_transposed_x_us": round(us_cols, 2),
            "rmsnorm_transposed_x_gbs": round(byts / (us_cols * 1e-6) / 1e9, 1),
            "fused_us": round(us_f, 1), "fused_with_norm_us": round(us_fn, 1),
            "fused_transposed_x_us": round(us_ft, 1), "fused_with_norm_transposed_x_us": round(us_fnt, 1),
            "timing": "cold: L2 and MALL flushed before each graph-replayed call",
        }), flush=True)
        del inp, x, xt, xn, ids, wts, out, ws
        torch.cuda.empty_cache()


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, w13, w2, T, budget_s):
    """The oracle (router + per-token FFN + combine, fp64) on the host cores,
    on a bounded sample of the same batch: batches of tokens from the start
    of the T-token batch until the time budget is spent (at least one
    batch), scaled to microseconds per call of T tokens."""
    import numpy as np
    import torch
    import oracle
    from mixture_experts_ffn_align_amd import workloads as W

    sh = inp["shape"]
    log("[bench] cpu baseline: copying weights to host")
    bits = lambda t: t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    g, u = W.packed_views(w13, sh.inter)
    G, U, D = bits(g), bits(u), bits(w2)
    x = bits(inp["x"])
    logits = inp["logits"].cpu().numpy()
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    oracle.lib()
    done = 0
    batch = max(threads, 4)
    t0 = time.perf_counter()
    while done == 0 or time.perf_counter() - t0 < budget_s:
        s0 = done % T
        n = min(batch, T - s0)
        ids, w = oracle.route(np.ascontiguousarray(logits[s0:s0 + n]), sh.routed_k)
        oracle.ffn(np.ascontiguousarray(x[s0:s0 + n]), ids, w, num_experts=sh.experts, gate=G, up=U,
                   w2=D)
        done += n
        if done % (4 * batch) == 0:
            log(f"[bench] cpu baseline: {done} tokens in {time.perf_counter() - t0:.1f} s")
    el = time.perf_counter() - t0
    return {
        "value": round(el / done * T * 1e6, 1),
        "unit": "us/call",
        "cores": threads,
        "kind": "oracle",
        "cpu": cpu_model(),
        "sample": f"{done} token-evaluations of the {T}-token batch (router + expert FFN + combine in fp64, "
                  f"{done / T:.2f} passes) in {el:.1f} s on {threads} threads, scaled to one call of {T} tokens",
    }


if __name__ == "__main__":
    main()
