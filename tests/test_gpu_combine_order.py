"""The combine's stated order, pinned bit for bit against an independent
emulation.

The library states its combine as acc = fmaf(w_tj, y_tj, acc) over the slots
j = 0 .. k-1 in order, from +0, with y_tj the bf16 per-slot row widened to
fp32, then one round to bf16 (the spec asks for a deterministic,
atomic-free combine that is bit-exact to a stated order). Here the per-slot
rows come out of the library through y_rows, and Python redoes that chain
exactly: each fmaf is the fp32 nearest to the exact w*y + acc (the product of
an fp32 and a bf16 value is exact in double; the sum is checked for
exactness with TwoSum and resolved with fractions where double rounded), and
the result must equal the fused call's out bit for bit. For the few-token
configurations whose gemm2 folds the combine in (no y in memory), y comes
from the configuration with the same K splits that writes it (the same MFMA
sequence per y element, tested bit-identical elsewhere).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import mixture_experts_ffn_align_amd as moe
from mixture_experts_ffn_align_amd import workloads as W
from harness import np_, np_bits, quantise_weights_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _f32_nearest(q: Fraction) -> np.float32:
    """fp32 nearest to an exact rational (ties to even), finite range."""
    f = np.float32(float(q))           # within one fp32 step of q
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(c)) - q)
        key = (d, int(np.array(c, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def _fmaf(w: np.ndarray, y: np.ndarray, acc: np.ndarray) -> np.ndarray:
    """Elementwise fp32 fma(w, y, acc) from float64 arrays holding fp32
    values (w, acc) and bf16 values (y)."""
    prod = w * y                       # exact: 24 + 8 significant bits
    s = prod + acc
    bb = s - prod
    err = (prod - (s - bb)) + (acc - bb)   # TwoSum: exact remainder of the double sum
    out = s.astype(np.float32)
    bad = np.nonzero(err != 0.0)
    for idx in zip(*bad):
        out[idx] = _f32_nearest(Fraction(float(prod[idx])) + Fraction(float(acc[idx])))
    return out.astype(np.float64)


def _bf16_bits_rne(v: np.ndarray) -> np.ndarray:
    u = v.astype(np.float32).view(np.uint32).astype(np.uint64)
    lower, upper = u & 0xFFFF, u >> 16
    up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    return ((upper + up) & 0xFFFF).astype(np.uint16)


def emulate_combine(y_bits: np.ndarray, ids: np.ndarray, w: np.ndarray, num_experts: int) -> np.ndarray:
    """out bits [T, H] from y_rows bits [T, k, H], ids and weights [T, k]."""
    T, k, H = y_bits.shape
    y = (y_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    acc = np.zeros((T, H), dtype=np.float64)
    for j in range(k):
        valid = (ids[:, j] >= 0) & (ids[:, j] < num_experts)
        nxt = _fmaf(w[:, j, None].astype(np.float64), y[:, j, :], acc)
        acc = np.where(valid[:, None], nxt, acc)
    return _bf16_bits_rne(acc)


def _y_rows(run, T, k, H):
    y = torch.full((T, k, H), float("nan"), dtype=torch.bfloat16, device=DEV)
    run(y)
    return np_bits(y)


@pytest.fixture(scope="module")
def w235():
    g = torch.Generator(device=DEV).manual_seed(1234)
    return W.draw_weights(W.QWEN3_235B_BF16, g, DEV)


@pytest.mark.parametrize("T", [512, 4, 1])
def test_bf16_combine_order(w235, T):
    sh = W.QWEN3_235B_BF16
    inp = W.make_inputs(sh, T, seed=40 + T, device=DEV, weights=w235)
    ids, w = moe.moe_topk_softmax(inp["logits"], sh.routed_k)
    gate, up = W.packed_views(inp["w13"], sh.inter)
    args = (inp["x"], gate, up, inp["w2"], ids, w)
    q = moe.moe_query_config(*args)
    cfg = q["config_index"]
    if q["gemm2_kernel"] == 6:
        # gemm2 folds the combine in: y from the weight streams with the same
        # 4-way K splits
        assert q["gemm1_split_k"] == 4 and q["gemm2_split_k"] == 4
        cfg = next(c for c in range(q["num_configs"]) if _splits(args, c) == (1, 2, 4, 4))
    out = np_bits(moe.moe_fused_fwd(*args))
    y = _y_rows(lambda y: moe.moe_fused_fwd(*args, y_rows=y, num_global_experts=sh.experts,
                                            force_config=cfg), T, sh.top_k, sh.hidden)
    want = emulate_combine(y, np_(ids), np_(w), sh.experts)
    assert (want == out).all(), f"{int((want != out).sum())} elements differ from the stated order"


def _splits(args, c, **kw):
    try:
        q = moe.moe_query_config(*args, force_config=c, **kw)
    except moe.MoEError:
        return None
    return (q["gemm1_kernel"] % 10, q["gemm2_kernel"] % 10, q["gemm1_split_k"], q["gemm2_split_k"])


@pytest.fixture(scope="module")
def fp4_513():
    sh = W.QWEN35_397B_TP2_FP4_513
    g = torch.Generator(device=DEV).manual_seed(78)
    w13, w2 = W.draw_weights(sh, g, DEV)
    q = quantise_weights_gpu(w13, w2, sh.inter)
    del w13, w2
    torch.cuda.empty_cache()
    return q


@pytest.mark.parametrize("T", [64, 2048, 4])
def test_mxfp4_combine_order(fp4_513, T):
    """513/11: eleven slots per token (the combine works in groups of 8, so
    the second group is covered), the shared expert at weight 1."""
    sh = W.QWEN35_397B_TP2_FP4_513
    (gq, gs), (uq, us), (wq, wsc) = fp4_513
    g = torch.Generator(device=DEV).manual_seed(T)
    x = torch.randn(T, sh.hidden, generator=g, device=DEV).to(torch.bfloat16)
    logits = torch.randn(T, sh.routed_experts, generator=g, device=DEV)
    ids, w = moe.moe_topk_softmax(logits, sh.routed_k, shared_id=sh.shared_expert, shared_w=1.0)
    kw = dict(gate_scale=gs, up_scale=us, w2_scale=wsc, mode=moe.MODE_MXFP4)
    args = (x, gq, uq, wq, ids, w)
    q = moe.moe_query_config(*args, **kw)
    cfg = q["config_index"]
    if q["gemm2_kernel"] == 16:
        want_splits = (q["gemm1_split_k"], q["gemm2_split_k"])
        cfg = next(c for c in range(q["num_configs"])
                   if (s := _splits(args, c, **kw)) is not None and s[1] in (2, 4) and s[2:] == want_splits)
    out = np_bits(moe.moe_fused_fwd(*args, **kw))
    y = _y_rows(lambda y: moe.moe_fused_fwd(*args, y_rows=y, num_global_experts=sh.experts, force_config=cfg,
                                            **kw), T, sh.top_k, sh.hidden)
    want = emulate_combine(y, np_(ids), np_(w), sh.experts)
    assert (want == out).all(), f"{int((want != out).sum())} elements differ from the stated order"


@pytest.mark.parametrize("lo,hi", [(-20, 21), (-140, -120)])
def test_combine_entry_point_order_with_skipped_slots(lo, hi):
    """moe_combine on strided rows with invalid ids, zero and negative
    weights, and magnitudes spread over 2^-20 .. 2^20 (so the fp32 sums
    round often), or down where products and sums are fp32 and bf16
    subnormals: the emulation of the stated order, bit for bit."""
    T, k, H, E = 37, 12, 512, 64
    g = torch.Generator(device=DEV).manual_seed(5)
    ybuf = torch.randn(T, k + 2, H, generator=g, device=DEV, dtype=torch.float64)
    ybuf *= torch.exp2(torch.randint(lo, hi, (T, k + 2, 1), generator=g, device=DEV).double())
    y = ybuf.to(torch.bfloat16)[:, 1:k + 1, :]   # rounded from fp64 (keeps bf16 subnormals)
    ids = torch.randint(-3, E + 3, (T, k), generator=g, device=DEV, dtype=torch.int32)
    w = torch.randn(T, k, generator=g, device=DEV)
    w[0, 0] = 0.0
    out = moe.moe_combine(y, ids, w, E)
    want = emulate_combine(np_bits(y.contiguous()), np_(ids), np_(w), E)
    assert (want == np_bits(out)).all()
