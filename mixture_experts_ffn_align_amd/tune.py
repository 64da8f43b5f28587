"""Per-bucket tile-configuration tuner for the fused forward.

The pages' tuned MXFP4 kernels come with a table of per-token-bucket choices
(block_m, kernel variant, measured latency and an error ratio against a
reference) that the dispatcher reads back (ROCm/aiter PR "TP2 MXFP4 fused-MoE
configs for Qwen3.5-397B", Details and the tuned latency table). This is the
same workflow for this library:

1. ``tune`` — for one layer shape and each token bucket T: draw the seeded
   synthetic inputs of that layer (workloads.py), route them, run every
   config index the library accepts for those sizes, gate each one's output
   against an independent reference of sampled tokens that the caller
   supplies (the pages' tuner checks every tuned kernel against a reference
   within errRatio 0.05, aiter PR, Details and Accuracy; here the rel-L2 and
   errRatio bounds of the layer's precision, and finite values), time the
   survivors as one call captured in a HIP graph and replayed back to back,
   and record the fastest in a CSV. Configs that split K like the built-in
   choice must also give its bits exactly (block_m and the kernel family
   never change a sum). For an expert-parallel shard (``ep`` > 1: experts
   [0, E/ep), global ids, per-slot rows out) only configs that split K like
   the unsharded call's choice are candidates, so shard rows stay
   bit-identical to it.
2. ``write_inc`` — merge CSVs into ``csrc/tuned_configs.inc``, the static
   table compiled into libmoeffn.so; ``moe_fused_fwd`` looks up the exact
   (mode, H, I, E, E_local, k, bucket) there before its built-in rules.

The reference comes from outside the library (the test suite's tuning driver
passes the CPU oracle), so this module itself only times and compares.

Usage (on a GPU, from the repository root):
    python tests/tune_gated.py --layer qwen3_235b_bf16 --buckets 1,2,4,...,32768 \\
        --out mixture_experts_ffn_align_amd/tuned/qwen3_235b_bf16.csv
    python -m mixture_experts_ffn_align_amd.tune --write-inc mixture_experts_ffn_align_amd/tuned/*.csv
then rebuild (mixture_experts_ffn_align_amd/build.py).
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import sys
import time
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
INC = os.path.join(HERE, "csrc", "tuned_configs.inc")
FIELDS = ["layer", "mode", "H", "I", "E", "E_local", "k", "bucket", "config", "us", "default_config",
          "default_us", "candidates", "rejected", "rel_l2", "err_ratio", "ref_tokens"]
GATES = {"bf16": (1e-2, 0.05), "mxfp4": (2e-2, 0.05)}   # (rel-L2, errRatio) bounds


def _layers():
    from . import workloads as W
    return {"tiny_bf16": W.TINY_BF16, "qwen3_235b_bf16": W.QWEN3_235B_BF16,
            "qwen35_397b_tp2_mxfp4_512": W.QWEN35_397B_TP2_FP4_512,
            "qwen35_397b_tp2_mxfp4_513": W.QWEN35_397B_TP2_FP4_513}


def _metrics(got, ref, rtol: float = 1e-2):
    """(rel-L2, errRatio, finite) of got against ref (float64 tensors or
    anything .double() accepts)."""
    import torch
    g, r = got.double(), torch.as_tensor(ref).double().to(got.device)
    finite = bool(torch.isfinite(g).all())
    rel = float((g - r).norm() / r.norm().clamp_min(1e-300))
    atol = rtol * float(r.pow(2).mean().sqrt())
    err = float(((g - r).abs() > rtol * r.abs() + atol).double().mean()) if g.numel() else 0.0
    return rel, err, finite


def _graph_us(call, budget_ms: float = 40.0, rounds: int = 2) -> float:
    """GPU microseconds per call: one call captured in a graph and replayed
    back to back for about budget_ms per round; the best of the rounds."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            call()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(reps):
        t0.record()
        for _ in range(reps):
            graph.replay()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e3 / reps

    one = timed(1)
    reps = max(3, min(400, int(budget_ms * 1e3 / max(one, 1.0))))
    us = min(timed(reps) for _ in range(rounds))
    del graph
    return us


def tune(layer: str, buckets, reference, ep: int = 1, seed: int = 0, log=print) -> list:
    """Tune one layer shape over token buckets; returns CSV rows (dicts).

    reference(T, x, ids, wts, weights) -> (toks, ref): the independent
    expected output rows ``ref`` [len(toks), H] (float64) of tokens ``toks``
    for this bucket's inputs, with the bf16 layer weights ``weights`` =
    (w13, w2) and, for an expert-parallel shard, slots of experts outside
    the shard dropped (ids set to -1). Candidates are gated on those rows."""
    import torch
    from . import workloads as W
    from . import (moe_fused_fwd, moe_fused_workspace_size, moe_query_config, moe_quant_mxfp4, moe_topk_softmax,
                   MODE_BF16, MODE_MXFP4)
    from . import MoEError

    sh = _layers()[layer]
    dev = torch.device("cuda")
    fp4 = sh.mode == "mxfp4"
    mode = MODE_MXFP4 if fp4 else MODE_BF16
    H, I, E, k = sh.hidden, sh.inter, sh.experts, sh.top_k
    if ep < 1 or E % ep:
        raise ValueError(f"ep = {ep} must divide E = {E}")
    es = E // ep
    g = torch.Generator(device=dev).manual_seed(seed)
    w13, w2 = W.draw_weights(sh, g, dev)
    gate, up = W.packed_views(w13, I)
    if fp4:
        (gq, gs), (uq, us_), (wq, ws_) = moe_quant_mxfp4(gate), moe_quant_mxfp4(up), moe_quant_mxfp4(w2)
        full_w = dict(gate=gq, up=uq, w2=wq, gate_scale=gs, up_scale=us_, w2_scale=ws_)
    else:
        full_w = dict(gate=gate, up=up, w2=w2)
    shard_w = {n: t[:es] for n, t in full_w.items()}
    rel_max, err_max = GATES[sh.mode]
    rows = []
    for T in buckets:
        inp = W.make_inputs(sh, T, seed=seed + T, device=dev, weights=(None, None))
        ids, wts = moe_topk_softmax(inp["logits"], sh.routed_k, True, sh.shared_expert, 1.0)
        x = inp["x"]

        def args(c, out=None, y=None, shard=True):
            wv = shard_w if shard else full_w
            kw = dict(gate_scale=wv.get("gate_scale"), up_scale=wv.get("up_scale"),
                      w2_scale=wv.get("w2_scale"), mode=mode, force_config=c)
            if ep > 1 and shard:
                kw.update(expert_offset=0, num_global_experts=E, y_rows=y)
            return (x, wv["gate"], wv["up"], wv["w2"], ids, wts), dict(kw, out=out)

        def query(c, shard=True):
            a, kw = args(c, shard=shard)
            if ep > 1 and shard:
                kw["y_rows"] = torch.empty((T, k, H), dtype=torch.bfloat16, device=dev)
                kw.pop("out")
            return moe_query_config(*a, **kw)

        base = query(-1)
        sig = None
        if ep > 1:
            full = query(-1, shard=False)
            sig = (full["gemm1_split_k"], full["gemm2_split_k"])
        cands = []
        for c in range(base["num_configs"]):
            try:
                q = query(c)
            except MoEError:
                continue
            if sig is not None and (q["gemm1_split_k"], q["gemm2_split_k"]) != sig:
                continue
            cands.append(c)

        def run(c):
            # each candidate gets its own workspace: its call is captured in
            # a graph for timing
            if ep > 1:
                y = torch.zeros((T, k, H), dtype=torch.bfloat16, device=dev)
                a, kw = args(c, y=y)
                kw.pop("out")
            else:
                out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
                a, kw = args(c, out=out)
            kw["workspace"] = torch.empty(moe_fused_workspace_size(*a, **kw), dtype=torch.uint8, device=dev)
            return lambda: moe_fused_fwd(*a, **kw)

        # the independent reference rows, and the candidates' rows of the
        # same tokens (a shard's per-slot rows summed over its own slots)
        ids_ref = ids
        if ep > 1:
            ids_ref = torch.where(ids < es, ids, torch.full_like(ids, -1))
        toks, ref_rows = reference(T, x, ids_ref, wts, (w13, w2))
        tsel = torch.as_tensor(toks, device=dev, dtype=torch.long)

        def rows_of(res):
            if ep > 1:
                y = res[tsel].double()                              # [n, k, H]
                wl = torch.where(ids_ref[tsel] >= 0, wts[tsel], torch.zeros_like(wts[tsel])).double()
                return (wl[:, :, None] * y).sum(1)
            return res[tsel]

        def splits(c):
            q = query(c)
            return (q["gemm1_split_k"], q["gemm2_split_k"])
        base_out = run(base["config_index"])().clone()
        timed, rejected = {}, []
        worst = (0.0, 0.0)
        for c in cands:
            call = run(c)
            got = call().clone()
            rel, err, finite = _metrics(rows_of(got), ref_rows)
            same_split = splits(c) == splits(base["config_index"])
            if not finite or rel > rel_max or err > err_max or (same_split and not torch.equal(got, base_out)):
                rejected.append(c)
                continue
            worst = (max(worst[0], rel), max(worst[1], err))
            timed[c] = _graph_us(call)
        if not timed:
            raise RuntimeError(f"{layer} T={T}: no config passed the reference gate (rejected {rejected})")
        best = min(timed, key=timed.get)
        row = {"layer": layer, "mode": mode, "H": H, "I": I, "E": E, "E_local": es, "k": k, "bucket": T,
               "config": best, "us": round(timed[best], 1), "default_config": base["config_index"],
               "default_us": round(timed.get(base["config_index"], float("nan")), 1),
               "candidates": len(cands), "rejected": " ".join(map(str, rejected)),
               "rel_l2": f"{worst[0]:.2e}", "err_ratio": f"{worst[1]:.2e}", "ref_tokens": len(toks)}
        log(f"[tune] {layer} ep{ep} T={T}: config {best} {row['us']} us "
            f"(built-in {row['default_config']} {row['default_us']} us; {len(timed)} timed, "
            f"{len(rejected)} rejected)")
        rows.append(row)
        del inp, ids, wts, x, base_out
        torch.cuda.empty_cache()
    return rows


def write_csv(rows, path: str) -> None:
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def read_csv(path: str) -> list:
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def write_inc(paths, inc: str = INC) -> int:
    """Merge tuned CSVs into the static table; later files win on equal keys."""
    table = {}
    for p in paths:
        for r in read_csv(p):
            key = tuple(int(r[n]) for n in ("mode", "H", "I", "E", "E_local", "k", "bucket"))
            table[key] = (int(r["config"]), float(r["us"]), r["layer"])
    lines = ["// Tuned tile configurations (written by mixture_experts_ffn_align_amd/tune.py).",
             "// mode, H, I, E (all shards), E_local, k, bucket, config index, us per call"]
    for key in sorted(table):
        c, us, layer = table[key]
        lines.append("{%d, %d, %d, %d, %d, %d, %d, %d, %.1ff},   // %s" % (*key, c, us, layer))
    with open(inc, "w") as f:
        f.write("\n".join(lines) + "\n")
    return len(table)


def add_tune_args(ap: argparse.ArgumentParser) -> None:
    ap.add_argument("--layer", choices=sorted(_layers()))
    ap.add_argument("--buckets", default=",".join(str(1 << i) for i in range(16)))
    ap.add_argument("--ep", type=int, default=1, help="expert-parallel shard 0 of this many")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--out", help="CSV to write")


def run_cli(a, reference) -> int:
    """Tune a.layer over a.buckets with ``reference`` as the gate; write a.out."""
    t0 = time.time()
    rows = tune(a.layer, [int(t) for t in a.buckets.split(",")], reference, ep=a.ep, seed=a.seed,
                log=lambda s: print(s, flush=True))
    write_csv(rows, a.out)
    print(f"[tune] {len(rows)} buckets in {time.time() - t0:.0f} s -> {a.out}", flush=True)
    return 0


def main(argv: Optional[list] = None) -> int:
    ap = argparse.ArgumentParser(description="merge tuned CSVs into the compiled-in table")
    ap.add_argument("--write-inc", nargs="*", metavar="CSV", required=True,
                    help="merge these CSVs into csrc/tuned_configs.inc (no GPU needed)")
    a = ap.parse_args(argv)
    paths = sorted(p for pat in a.write_inc for p in glob.glob(pat))
    n = write_inc(paths)
    print(f"[tune] wrote {n} rows to {INC}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
