"""Helpers shared by the GPU parity tests: run the HIP path through the
binding, run the oracle on the same bytes, and compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import mixture_experts_ffn_align_amd as moe
from mixture_experts_ffn_align_amd import workloads as W

RTOL = 1e-2


def np_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor on any device -> numpy uint16 bit patterns (strides kept on CPU)."""
    if t.device.type != "cpu":
        t = t.cpu()
    return t.view(torch.int16).numpy().view(np.uint16)


def np_(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy() if t.device.type != "cpu" else t.numpy()


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def err_ratio(got: np.ndarray, ref: np.ndarray, rtol: float = RTOL) -> float:
    """Fraction of elements with |got - ref| > rtol*|ref| + rtol*rms(ref)."""
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    atol = rtol * float(np.sqrt(np.mean(ref * ref)))
    bad = np.abs(got - ref) > rtol * np.abs(ref) + atol
    return float(bad.mean())


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def sample_tokens(T: int, n: int = 8, seed: int = 0) -> np.ndarray:
    if T <= n:
        return np.arange(T, dtype=np.int64)
    rng = np.random.default_rng(seed + T)
    pick = {0, T - 1, T // 2}
    while len(pick) < n:
        pick.add(int(rng.integers(0, T)))
    return np.array(sorted(pick), dtype=np.int64)


def tail_tokens(ids: np.ndarray, num_experts: int, n: int, seed: int = 0) -> np.ndarray:
    """At least ``n`` tokens (all of them if T <= n) that include, for every
    expert with assignments, the token of its last assignment in flat order
    t*k + j. The align puts an expert's assignments in ascending flat order,
    so that token sits in the expert's last (ragged, sentinel-padded) sorted
    block whatever block_m is; the rest are the first, middle and last
    tokens and seeded random ones."""
    T, k = ids.shape
    if T <= n:
        return np.arange(T, dtype=np.int64)
    flat = np.ascontiguousarray(ids).reshape(-1).astype(np.int64)
    ok = (flat >= 0) & (flat < num_experts)
    last = np.full(num_experts, -1, dtype=np.int64)
    np.maximum.at(last, flat[ok], np.arange(flat.size, dtype=np.int64)[ok])
    pick = set(int(a) // k for a in last[last >= 0]) | {0, T // 2, T - 1}
    rng = np.random.default_rng(seed + T)
    while len(pick) < n:
        pick.add(int(rng.integers(0, T)))
    return np.array(sorted(pick), dtype=np.int64)


def route_both(inp: dict):
    """(gpu ids, gpu w) from the HIP router; (oracle ids, oracle w) from the oracle."""
    sh: W.MoEShape = inp["shape"]
    logits = inp["logits"]
    shared = sh.shared_expert
    gi, gw = moe.moe_topk_softmax(logits, sh.routed_k, True, shared, 1.0)
    oi, ow = oracle.route(np_(logits).astype(np.float32), sh.routed_k, True, shared, 1.0)
    return (gi, gw), (oi, ow)


def assert_routing_equal(g, o):
    gi, gw = np_(g[0]), np_(g[1])
    oi, ow = o
    assert gi.shape == oi.shape
    assert (gi == oi).all(), "router ids differ from the oracle"
    bad = int((gw.view(np.int32) != ow.view(np.int32)).sum())
    assert bad == 0, f"{bad} router weights differ from the oracle's bits"


def quantise_weights_gpu(w13: torch.Tensor, w2: torch.Tensor, inter: int):
    gate, up = W.packed_views(w13, inter)
    gq = moe.moe_quant_mxfp4(gate)
    uq = moe.moe_quant_mxfp4(up)
    wq = moe.moe_quant_mxfp4(w2)
    return gq, uq, wq


def oracle_quant_experts(w13: torch.Tensor, w2: torch.Tensor, inter: int, experts) -> dict:
    """Oracle-side MXFP4 codes of the listed experts' gate, up and w2."""
    out = {}
    for e in experts:
        g = np_bits(w13[e, :inter, :])
        u = np_bits(w13[e, inter:, :])
        d = np_bits(w2[e])
        out[e] = (oracle.mxfp4_quant(g), oracle.mxfp4_quant(u), oracle.mxfp4_quant(d))
    return out


def oracle_ffn_tokens(inp: dict, ids: np.ndarray, w: np.ndarray, toks: np.ndarray,
                      gate=None, up=None, mx=None):
    """Oracle output rows for tokens ``toks``.

    bf16 mode: gate/up default to the packed views of inp["w13"].
    MXFP4 mode: ``mx`` maps expert -> oracle codes from oracle_quant_experts;
    other experts are given zero codes (the listed tokens never use them).
    """
    sh: W.MoEShape = inp["shape"]
    E, I, H = sh.experts, sh.inter, sh.hidden
    x = np_bits(inp["x"])
    ids_s = np.ascontiguousarray(ids[toks])
    w_s = np.ascontiguousarray(w[toks])
    x_s = np.ascontiguousarray(x[toks])
    if mx is None:
        if gate is None:
            gate, up = W.packed_views(inp["w13"], I)
        used = sorted({int(e) for e in ids_s.ravel() if 0 <= e < E})
        # compact the experts the tokens use, keeping ids consistent
        remap = {e: i for i, e in enumerate(used)}
        ids_c = np.vectorize(lambda e: remap.get(int(e), -1))(ids_s).astype(np.int32) if used else \
            np.full_like(ids_s, -1)
        g = np.stack([np_bits(gate[e]) for e in used]) if used else np.zeros((0, I, H), np.uint16)
        u = np.stack([np_bits(up[e]) for e in used]) if used else np.zeros((0, I, H), np.uint16)
        d = np.stack([np_bits(inp["w2"][e]) for e in used]) if used else np.zeros((0, H, I), np.uint16)
        acc, ob = oracle.ffn(x_s, ids_c, w_s, num_experts=max(len(used), 1), gate=g, up=u, w2=d)
        return acc, ob
    used = sorted({int(e) for e in ids_s.ravel() if 0 <= e < E})
    remap = {e: i for i, e in enumerate(used)}
    ids_c = np.vectorize(lambda e: remap.get(int(e), -1))(ids_s).astype(np.int32)
    parts = [[mx[e][p][q] for e in used] for p in range(3) for q in range(2)]
    gq = (np.stack(parts[0]), np.stack(parts[1]))
    uq = (np.stack(parts[2]), np.stack(parts[3]))
    wq = (np.stack(parts[4]), np.stack(parts[5]))
    return oracle.ffn(x_s, ids_c, w_s, num_experts=len(used), gate_q=gq, up_q=uq, w2_q=wq)
