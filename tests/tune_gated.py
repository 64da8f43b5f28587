"""The tile-config tuner gated on the CPU oracle.

The library's tuner (mixture_experts_ffn_align_amd/tune.py) times every
config per token bucket and keeps the fastest one that passes a reference
gate; the reference has to come from outside the library, so this driver
supplies the oracle: for each bucket, the oracle's output rows of a seeded
sample of tokens that includes tokens from the experts' ragged last sorted
blocks, computed from the bf16 weights (MXFP4 layers: quantised by the
oracle's own MXFP4 routine). The pages' tuner gates every tuned kernel the
same way, against a reference within errRatio 0.05 (ROCm/aiter PR "TP2
MXFP4 fused-MoE configs for Qwen3.5-397B", Details and Accuracy).

Usage (GPU, repository root):
    python tests/tune_gated.py --layer qwen3_235b_bf16 --buckets 1,2,...,32768 --out <csv>
then merge with ``python -m mixture_experts_ffn_align_amd.tune --write-inc <csvs>``.
"""
from __future__ import annotations

import argparse
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

import numpy as np  # noqa: E402

from harness import np_, oracle_ffn_tokens, oracle_quant_experts  # noqa: E402
from mixture_experts_ffn_align_amd import tune  # noqa: E402


def gate_tokens(ids: np.ndarray, num_experts: int, n: int, seed: int = 0) -> np.ndarray:
    """n tokens (all if T <= n): tokens holding experts' last assignments
    (in their ragged last sorted block) first, then seeded random ones."""
    T, k = ids.shape
    if T <= n:
        return np.arange(T, dtype=np.int64)
    flat = np.ascontiguousarray(ids).reshape(-1).astype(np.int64)
    ok = (flat >= 0) & (flat < num_experts)
    last = np.full(num_experts, -1, dtype=np.int64)
    np.maximum.at(last, flat[ok], np.arange(flat.size, dtype=np.int64)[ok])
    tails = np.unique(last[last >= 0] // k)
    rng = np.random.default_rng(seed + T)
    pick = set(rng.choice(tails, size=min(n // 2, tails.size), replace=False).tolist())
    while len(pick) < n:
        pick.add(int(rng.integers(0, T)))
    return np.array(sorted(pick), dtype=np.int64)


def oracle_reference(layer: str, n_tokens: int = 24, scale: float = 1.0):
    """reference(T, x, ids, wts, (w13, w2)) for tune.tune, from the oracle.
    ``scale`` multiplies the reference (1.0 for real use; tests plant a
    mistake with another value to show the gate rejects)."""
    sh = tune._layers()[layer]
    memo = {}

    def reference(T, x, ids, wts, weights):
        w13, w2 = weights
        oi, ow = np_(ids), np_(wts)
        toks = gate_tokens(oi, sh.experts, n_tokens)
        inp = {"shape": sh, "x": x, "w13": w13, "w2": w2}
        if sh.mode == "mxfp4":
            used = sorted({int(e) for e in oi[toks].ravel() if 0 <= e < sh.experts})
            missing = [e for e in used if e not in memo]
            if missing:
                memo.update(oracle_quant_experts(w13, w2, sh.inter, missing))
            acc, _ = oracle_ffn_tokens(inp, oi, ow, toks, mx={e: memo[e] for e in used})
        else:
            acc, _ = oracle_ffn_tokens(inp, oi, ow, toks)
        return toks, acc * scale
    return reference


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description="tune tile configs per bucket, gated on the CPU oracle")
    tune.add_tune_args(ap)
    ap.add_argument("--ref-tokens", type=int, default=24)
    a = ap.parse_args(argv)
    if not a.layer or not a.out:
        ap.error("--layer and --out are required")
    return tune.run_cli(a, oracle_reference(a.layer, a.ref_tokens))


if __name__ == "__main__":
    sys.exit(main())
