#!/usr/bin/env python3
"""Benchmark of the fused MoE expert-FFN forward on one MI355X.

One step = the whole hot path on one batch: router (top-k softmax) and the
fused forward (align, gemm1 + SiLU*up, gemm2, combine) for the
Qwen3-235B-shaped bf16 layer (H=4096, I=1536, E=128, top-8) at T=512 tokens,
gate/up passed as views into the packed w13. Inputs are seeded synthetic
tensors already resident in HBM. The JSON line also carries the same layer at
T=4096 and T=16384 with router-replay id slices (the other token counts the
metric names), the per-stage times from HIP events, the roofline of the
dominant kernel (gemm1) and the oracle timed on the host cores.

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
KERNEL_FAMILY = {1: "gemm_stream", 3: "gemm_tile", 11: "gemm_stream", 13: "gemm_tile"}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget for the oracle's CPU baseline sample (0 to skip)")
    ap.add_argument("--no-extra", action="store_true", help="skip the T=4096/16384 lines")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy three times (counter calibration)")
    ap.add_argument("--mxfp4", default="",
                    help="comma-separated token buckets: instead of the bf16 line, one JSON line per "
                         "bucket for the MXFP4 TP2 shard (E=512, top-10)")
    ap.add_argument("--bf16", default="",
                    help="comma-separated token buckets: one JSON line per bucket for the bf16 "
                         "Qwen3-235B-shaped layer (graph-timed fused forward, packed w13 views)")
    ap.add_argument("--ep", type=int, default=0,
                    help="with --bf16: time one expert-parallel shard of S (experts [0, E/S), global "
                         "ids, per-slot rows out) and the tokens' home combine instead of the whole layer")
    ap.add_argument("--norm", default="",
                    help="comma-separated token counts: the RMSNorm pre-pass on its own (contiguous and "
                         "transposed x) and inside the bf16 fused forward, one JSON line each")
    ap.add_argument("--bwd", default="",
                    help="comma-separated token counts: the backward of the bf16 Qwen3-235B-shaped layer "
                         "(fp32 weight gradients), one JSON line each")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(multi-GPU expert/tensor parallel sharding is a design note, not built).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import mixture_experts_ffn_align_amd as moe
    from mixture_experts_ffn_align_amd import workloads as W

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
        mxfp4_buckets([int(t) for t in args.mxfp4.split(",")], args, dev)
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
        bf16_buckets([int(t) for t in args.bf16.split(",")], args, dev)
        return
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
    gpu_ms = 0.0
    for evs in evsets:
        stage_ms["route"] += hip.elapsed_ms(evs[0], evs[1])
        for s, name in enumerate(moe.STAGES):
            stage_ms[name] += hip.elapsed_ms(evs[2 + 2 * s], evs[3 + 2 * s])
        gpu_ms += hip.elapsed_ms(evs[0], evs[-1])
    for key in stage_ms:
        stage_ms[key] /= args.steps
    gpu_ms /= args.steps
    for evs in evsets:
        hip.destroy(evs)

    touched = int(torch.unique(ids).numel())
    A = T * k
    per_expert = 3 * I * H * 2
    bytes_call = touched * per_expert + 2 * T * H * 2 + 8 * A + T * sh.routed_experts * 4
    flops_call = 6 * H * I * A
    us = ms_per_step * 1e3
    tflops = flops_call / (us * 1e-6) / 1e12
    roof_call = max(bytes_call / (HBM_PEAK_GBS * 1e9), flops_call / (BF16_PEAK_TFLOPS * 1e12)) / (us * 1e-6)
    g1_bytes = touched * 2 * I * H * 2 + T * H * 2
    g1_s = g1_live_ms * 1e-3
    g1_gbs = g1_bytes / g1_s / 1e9
    traffic = read_traffic()

    # flushed single calls: a 512 MB write before each call evicts L2 and MALL
    flush = torch.empty(512 * 2 ** 20 // 4, dtype=torch.float32, device=dev)
    flushed = []
    e2 = hip.create(2)
    for _ in range(10):
        flush.fill_(1.0)
        hip.record(e2[0], stream)
        step()
        hip.record(e2[1], stream)
        torch.cuda.synchronize()
        flushed.append(hip.elapsed_ms(e2[0], e2[1]))
    del flush
    flushed_us = float(np.median(flushed)) * 1e3

    extra = {}
    if not args.no_extra:
        for TT in (4096, 16384):
            log(f"[bench] T={TT} router-replay slices, packed views")
            ri = W.make_inputs(sh, TT, seed=0, device=dev, routing="replay", weights=(w13, w2))
            xo = torch.empty(TT, H, dtype=torch.bfloat16, device=dev)
            ids_s, w_s = ri["topk_ids"], ri["topk_weights"]
            wsx = torch.empty(moe.moe_fused_workspace_size(ri["x"], gate, up, w2, ids_s, w_s),
                              dtype=torch.uint8, device=dev)
            n_w, n_t = max(3, args.warmup // 2), max(5, args.steps // 4)
            for _ in range(n_w):
                moe.moe_fused_fwd(ri["x"], gate, up, w2, ids_s, w_s, out=xo, workspace=wsx, stream=stream)
            ev = hip.create(2 + 2 * nst)
            g1 = g2 = 0.0
            torch.cuda.synchronize()
            ta = time.perf_counter()
            for _ in range(n_t):
                moe.moe_fused_fwd(ri["x"], gate, up, w2, ids_s, w_s, out=xo, workspace=wsx,
                                  stage_events=ev[2:], stream=stream)
                torch.cuda.synchronize()
                g1 += hip.elapsed_ms(ev[2 + 2 * 2], ev[3 + 2 * 2])
                g2 += hip.elapsed_ms(ev[2 + 2 * 3], ev[3 + 2 * 3])
            tb = time.perf_counter()
            hip.destroy(ev)
            qt = moe.moe_query_config(ri["x"], gate, up, w2, ids_s, w_s)
            us_t = (tb - ta) * 1e6 / n_t
            At = TT * k
            touched_t = int(torch.unique(ids_s).numel())
            b_t = touched_t * per_expert + 2 * TT * H * 2 + 8 * At
            f_t = 6 * H * I * At
            extra[str(TT)] = {
                "us_per_call": round(us_t, 1),
                "tflops": round(f_t / (us_t * 1e-6) / 1e12, 1),
                "roofline_frac": round(max(b_t / (HBM_PEAK_GBS * 1e9), f_t / (BF16_PEAK_TFLOPS * 1e12))
                                       / (us_t * 1e-6), 3),
                "bound": "hbm" if b_t / HBM_PEAK_GBS / 1e9 > f_t / BF16_PEAK_TFLOPS / 1e12 else "mfma",
                "gemm1_us": round(g1 * 1e3 / n_t, 1),
                "gemm2_us": round(g2 * 1e3 / n_t, 1),
                # MFMA utilisation of the GEMMs alone (algorithmic flops over their time)
                "gemm1_mfma_frac": round(4 * H * I * At / (g1 * 1e-3 / n_t) / (BF16_PEAK_TFLOPS * 1e12), 3),
                "gemm2_mfma_frac": round(2 * H * I * At / (g2 * 1e-3 / n_t) / (BF16_PEAK_TFLOPS * 1e12), 3),
                "kernel": f"{KERNEL_FAMILY.get(qt['gemm1_kernel'], '?')} block_m={qt['block_m']}",
                "inputs": "packed w13 views, ids/weights [:, :, 7, :] of [1,T,46,8] (token stride 368)",
            }
            del ri, xo, wsx
            torch.cuda.empty_cache()

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
        "tflops": round(tflops, 2),
        "roofline_frac_call": round(roof_call, 3),
        "touched_experts": touched,
        "algorithmic_bytes_per_call": bytes_call,
        "gpu_us_per_step_events": round(gpu_ms * 1e3, 1),
        "flushed_us_per_call_median": round(flushed_us, 1),
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
        "per_tokens": extra,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def graph_time_us(call, reps):
    """One call captured in a HIP graph, replayed back to back: GPU time per
    call (the eager result is checked against the replay first)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            out = call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = call()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    if not torch.equal(out, eager):
        raise RuntimeError("graph replay differs from the eager call")
    hip = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    ev = hip.create(2)
    hip.record(ev[0], stream)
    for _ in range(reps):
        graph.replay()
    hip.record(ev[1], stream)
    torch.cuda.synchronize()
    us = hip.elapsed_ms(ev[0], ev[1]) * 1e3 / reps
    hip.destroy(ev)
    del graph
    return us


def bf16_buckets(buckets, args, dev):
    """bf16 Qwen3-235B-shaped layer (H=4096, I=1536, E=128, top-8): per token
    bucket, the fused forward on router ids computed beforehand, gate/up as
    packed w13 views, graph-timed."""
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
    for T in buckets:
        inp = W.make_inputs(sh, T, seed=T, device=dev, weights=(w13, w2))
        ids, wts = moe.moe_topk_softmax(inp["logits"], k)
        out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        ws = torch.empty(moe.moe_fused_workspace_size(inp["x"], gate, up, w2, ids, wts), dtype=torch.uint8,
                         device=dev)
        cfg = moe.moe_query_config(inp["x"], gate, up, w2, ids, wts)
        reps = max(5, min(200, int(2e5 / (T + 50))))
        us_call = graph_time_us(lambda: moe.moe_fused_fwd(inp["x"], gate, up, w2, ids, wts, out=out, workspace=ws),
                                reps)
        touched = int(torch.unique(ids).numel())
        A = T * k
        byts = touched * per_expert + T * H * 2 * 2 + 8 * A
        flops = 6 * H * I * A
        hbm_s, mfma_s = byts / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12)
        print(json.dumps({
            "workload": f"{sh.name}, fused forward on given top-k ids/weights, packed w13 views",
            "tokens": T, "touched_experts": touched, "us_per_call": round(us_call, 1),
            "timing": f"HIP graph of one call, {reps} replays back to back",
            "algorithmic_bytes": byts, "tflops": round(flops / (us_call * 1e-6) / 1e12, 2),
            "bound": "hbm" if hbm_s >= mfma_s else "mfma",
            "roofline_frac": round(max(hbm_s, mfma_s) / (us_call * 1e-6), 3),
            "hbm_gbs": round(byts / (us_call * 1e-6) / 1e9, 1),
            "config": {kk: cfg[kk] for kk in ("config_index", "block_m", "block_m2", "gemm1_kernel",
                                               "gemm2_kernel", "gemm1_split_k", "gemm2_split_k")},
        }), flush=True)
        del inp, ids, wts, out, ws
        torch.cuda.empty_cache()


def ep_buckets(buckets, S, dev):
    """One expert-parallel shard of the bf16 Qwen3-235B-shaped layer: shard 0
    of S holds experts [0, E/S) as views into packed w13, takes the global
    top-8 ids, and writes the per-slot rows of its slots (what an all-to-all
    would return to the tokens' home ranks); then the home combine of all T*k
    rows. Both graph-timed; inputs as in --bf16."""
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
    for T in buckets:
        inp = W.make_inputs(sh, T, seed=T, device=dev, weights=(w13, w2))
        ids, wts = moe.moe_topk_softmax(inp["logits"], k)
        y = torch.zeros((T, k, H), dtype=torch.bfloat16, device=dev)   # foreign rows stay 0
        out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        kw = dict(expert_offset=0, num_global_experts=E, y_rows=y)
        ws = torch.empty(moe.moe_fused_workspace_size(inp["x"], gs, us, w2s, ids, wts, **kw),
                         dtype=torch.uint8, device=dev)
        reps = max(5, min(200, int(2e5 / (T / S + 50))))
        us_shard = graph_time_us(lambda: moe.moe_fused_fwd(inp["x"], gs, us, w2s, ids, wts, workspace=ws, **kw),
                                 reps)
        us_comb = graph_time_us(lambda: moe.moe_combine(y, ids, wts, E, out=out), reps)
        local = (ids < es)
        n_local = int(local.sum().item())
        touched = int(torch.unique(ids[local]).numel())
        byts = touched * per_expert + T * H * 2 + n_local * H * 2 + 4 * T * k
        flops = 6 * H * I * n_local
        hbm_s, mfma_s = byts / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12)
        comb_bytes = T * k * H * 2 + T * H * 2 + 8 * T * k
        print(json.dumps({
            "workload": f"{sh.name}, expert-parallel shard 0 of {S} (experts [0, {es})), global ids, "
                        "per-slot rows out; then the home combine of all rows",
            "tokens": T, "local_slots": n_local, "touched_local_experts": touched,
            "shard_us_per_call": round(us_shard, 1),
            "shard_algorithmic_bytes": byts,
            "shard_bound": "hbm" if hbm_s >= mfma_s else "mfma",
            "shard_roofline_frac": round(max(hbm_s, mfma_s) / (us_shard * 1e-6), 3),
            "shard_hbm_gbs": round(byts / (us_shard * 1e-6) / 1e9, 1),
            "combine_us_per_call": round(us_comb, 1),
            "combine_hbm_gbs": round(comb_bytes / (us_comb * 1e-6) / 1e9, 1),
            "timing": f"HIP graph of one call, {reps} replays back to back",
        }), flush=True)
        del inp, ids, wts, y, out, ws
        torch.cuda.empty_cache()


def bwd_lines(tokens, dev):
    """Backward of the bf16 Qwen3-235B-shaped layer: gradients of sum(dout * out)
    for x, the top-k weights and all three weight tensors (fp32), one call
    graph-timed, with the weight gradients overwritten and with them
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
        reps = max(3, min(50, int(5e4 / (T + 50))))
        us = graph_time_us(call, reps)
        us_acc = graph_time_us(lambda: call(True), reps)
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
            "timing": f"HIP graph of one call, {reps} replays back to back",
        }), flush=True)
        del inp, ids, wts, dout, dx, dwt, ws
        torch.cuda.empty_cache()


def norm_lines(tokens, dev):
    """RMSNorm of H=4096 bf16 rows (weight fp32 uniform [0, 1), eps 1e-6):
    moe_rmsnorm on a contiguous and on a transposed x, and the bf16
    Qwen3-235B-shaped fused forward with and without norm_weight. Graph-timed."""
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
    for T in tokens:
        inp = W.make_inputs(sh, T, seed=T, device=dev, weights=(w13, w2))
        x = inp["x"]
        xt = x.t().contiguous().t()
        xn = torch.empty_like(x)
        ids, wts = moe.moe_topk_softmax(inp["logits"], k)
        out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        ws = torch.empty(moe.moe_fused_workspace_size(x, gate, up, w2, ids, wts, norm_weight=nw),
                         dtype=torch.uint8, device=dev)
        reps = max(5, min(200, int(2e6 / (T + 50))))
        us_rows = graph_time_us(lambda: moe.moe_rmsnorm(x, nw, 1e-6, out=xn), reps)
        us_cols = graph_time_us(lambda: moe.moe_rmsnorm(xt, nw, 1e-6, out=xn), reps)
        fr = max(5, min(100, int(2e5 / (T + 50))))
        us_f = graph_time_us(lambda: moe.moe_fused_fwd(x, gate, up, w2, ids, wts, out=out, workspace=ws), fr)
        us_fn = graph_time_us(lambda: moe.moe_fused_fwd(x, gate, up, w2, ids, wts, out=out, workspace=ws,
                                                        norm_weight=nw, norm_eps=1e-6), fr)
        byts = T * H * 2 * 2 + H * 4
        print(json.dumps({
            "workload": f"RMSNorm of [T, {H}] bf16 rows, fp32 weight; {sh.name} fused forward with it",
            "tokens": T,
            "rmsnorm_us": round(us_rows, 2), "rmsnorm_gbs": round(byts / (us_rows * 1e-6) / 1e9, 1),
            "rmsnorm_hbm_frac": round(byts / (us_rows * 1e-6) / 1e9 / HBM_PEAK_GBS, 3),
            "rmsnorm_transposed_x_us": round(us_cols, 2),
            "rmsnorm_transposed_x_gbs": round(byts / (us_cols * 1e-6) / 1e9, 1),
            "fused_us": round(us_f, 1), "fused_with_norm_us": round(us_fn, 1),
            "timing": "HIP graph of one call, replayed back to back",
        }), flush=True)
        del inp, x, xt, xn, ids, wts, out, ws
        torch.cuda.empty_cache()


def mxfp4_buckets(buckets, args, dev):
    """MXFP4 TP2 shard (H=4096, I=512, E=512, top-10): per token bucket, the
    fused forward (align + activation quantisation, gemm1 + SiLU*up with h
    quantised, gemm2, combine) on router ids/weights already computed. A call
    is captured once in a HIP graph and replayed back to back, so the time is
    the GPU's, not the host's argument marshalling; the stage split comes from
    a separate eager pass with HIP events (about 2 us of marker cost each)."""
    import torch
    import mixture_experts_ffn_align_amd as moe
    from mixture_experts_ffn_align_amd import workloads as W

    sh = W.QWEN35_397B_TP2_FP4_512
    H, I, E, k = sh.hidden, sh.inter, sh.experts, sh.top_k
    log(f"[bench] drawing and quantising weights {sh.name}")
    g = torch.Generator(device=dev).manual_seed(0)
    w13, w2 = W.draw_weights(sh, g, dev)
    gate, up = W.packed_views(w13, I)
    (gq, gs), (uq, us), (wq, wsc) = moe.moe_quant_mxfp4(gate), moe.moe_quant_mxfp4(up), moe.moe_quant_mxfp4(w2)
    del w13, w2, gate, up
    torch.cuda.empty_cache()
    hip = HipEvents()
    nst = len(moe.STAGES)
    per_expert = 3 * I * H // 2 + 3 * I * H // 32          # e2m1 codes + e8m0 scales of gate, up, down
    for T in buckets:
        gx = torch.Generator(device=dev).manual_seed(T)
        x = torch.randn(T, H, generator=gx, device=dev).to(torch.bfloat16)
        logits = torch.randn(T, E, generator=gx, device=dev)
        ids, wts = moe.moe_topk_softmax(logits, k)
        out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        kw = dict(gate_scale=gs, up_scale=us, w2_scale=wsc, mode=moe.MODE_MXFP4)
        ws = torch.empty(moe.moe_fused_workspace_size(x, gq, uq, wq, ids, wts, **kw), dtype=torch.uint8, device=dev)
        cfg = moe.moe_query_config(x, gq, uq, wq, ids, wts, **kw)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):                       # warm up off the capture
            for _ in range(3):
                moe.moe_fused_fwd(x, gq, uq, wq, ids, wts, out=out, workspace=ws, **kw)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        eager = out.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            moe.moe_fused_fwd(x, gq, uq, wq, ids, wts, out=out, workspace=ws, **kw)
        reps = max(5, min(200, int(2e5 / (T + 50))))
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, eager):
            raise RuntimeError(f"T={T}: graph replay differs from the eager call")
        stream = torch.cuda.current_stream().cuda_stream
        ev = hip.create(2)
        hip.record(ev[0], stream)
        for _ in range(reps):
            graph.replay()
        hip.record(ev[1], stream)
        torch.cuda.synchronize()
        us_call = hip.elapsed_ms(ev[0], ev[1]) * 1e3 / reps
        hip.destroy(ev)
        del graph
        evs = hip.create(2 * nst)
        st = {s: [] for s in moe.STAGES}
        for _ in range(10):
            moe.moe_fused_fwd(x, gq, uq, wq, ids, wts, out=out, workspace=ws, stage_events=evs, stream=stream, **kw)
            torch.cuda.synchronize()
            for i, s in enumerate(moe.STAGES):
                st[s].append(hip.elapsed_ms(evs[2 * i], evs[2 * i + 1]) * 1e3)
        hip.destroy(evs)
        touched = int(torch.unique(ids).numel())
        A = T * k
        byts = touched * per_expert + T * H * 2 * 2 + 8 * A
        flops = 6 * H * I * A
        hbm_s, mfma_s = byts / (HBM_PEAK_GBS * 1e9), flops / (FP4_PEAK_TFLOPS * 1e12)
        line = {
            "workload": f"{sh.name}, fused forward on given top-k ids/weights",
            "tokens": T, "touched_experts": touched, "us_per_call": round(us_call, 1),
            "timing": f"HIP graph of one call, {reps} replays back to back",
            "algorithmic_bytes": byts, "tflops": round(flops / (us_call * 1e-6) / 1e12, 2),
            "bound": "hbm" if hbm_s >= mfma_s else "mfma",
            "roofline_frac": round(max(hbm_s, mfma_s) / (us_call * 1e-6), 3),
            "hbm_gbs": round(byts / (us_call * 1e-6) / 1e9, 1),
            "stage_us_eager_events": {s: round(sorted(v)[len(v) // 2], 1) for s, v in st.items()},
            "config": {kk: cfg[kk] for kk in ("config_index", "block_m", "block_m2", "gemm1_kernel",
                                               "gemm2_kernel", "gemm1_split_k", "gemm2_split_k")},
        }
        print(json.dumps(line), flush=True)
        del x, logits, ids, wts, out, ws
        torch.cuda.empty_cache()


def cpu_baseline(inp, w13, w2, T, budget_s):
    """The oracle (router + per-token FFN + combine, fp64) on the host cores,
    on the same batch: whole passes over the T tokens until the time budget
    is spent (at least one pass; the last pass may stop early), scaled to
    microseconds per call of T tokens."""
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
    while done < T or time.perf_counter() - t0 < budget_s:
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
        "sample": f"{done} token-evaluations ({done / T:.2f} passes over the {T}-token batch: router + "
                  f"expert FFN + combine in fp64) in {el:.1f} s on {threads} threads, scaled to one "
                  f"call of {T} tokens",
    }


if __name__ == "__main__":
    main()
