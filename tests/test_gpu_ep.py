"""Expert-parallel shards on one GPU.

One MI355X stands in for each rank of an expert-parallel group in turn: a
shard call gets the weights of experts [o, o + E_s) as views into the full
tensors, the global top-k ids, ``expert_offset = o`` and the global expert
count. Checked here:

* every shard writes the per-slot results of its own slots into one
  [T, k, H] buffer (the rows an all-to-all would send home), and
  ``moe_combine`` over that buffer gives the unsharded call's output bit for
  bit, in bf16 and MXFP4, with uniform and Zipf-skewed routing (some shards
  then own experts that receive no tokens);
* rows of other shards' slots are left untouched;
* a shard that combines into ``out`` itself equals the unsharded call with
  the other shards' ids replaced by an invalid id (bit for bit), and the
  oracle on the shard's experts (bf16 rel-L2 <= 1e-2).
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_align_amd as moe
from mixture_experts_ffn_align_amd import workloads as W
from harness import (bf16_to_f64, np_, np_bits, oracle_ffn_tokens, quantise_weights_gpu, rel_l2,
                     route_both, sample_tokens)

pytestmark = pytest.mark.gpu
DEV = "cuda"
FILL = 0x7FC1          # a NaN pattern no shard ever writes


@pytest.fixture(scope="module")
def w235():
    g = torch.Generator(device=DEV).manual_seed(4321)
    return W.draw_weights(W.QWEN3_235B_BF16, g, DEV)


def _shards(E, S):
    es = E // S
    return [(s * es, es) for s in range(S)]


def _bits(t):
    return np_bits(t.contiguous())


@pytest.mark.parametrize("T,kind", [(1, "uniform"), (7, "zipf"), (512, "uniform"), (4096, "uniform"), (4099, "zipf")])
def test_bf16_ep8_rows_combine_to_unsharded(w235, T, kind):
    sh = W.QWEN3_235B_BF16
    inp = W.make_inputs(sh, T, seed=50 + T, device=DEV, weights=w235, logits_kind=kind)
    (ids, w), _ = route_both(inp)
    gate, up = W.packed_views(inp["w13"], sh.inter)
    full = moe.moe_fused_fwd(inp["x"], gate, up, inp["w2"], ids, w)
    y = torch.empty((T, sh.top_k, sh.hidden), dtype=torch.bfloat16, device=DEV)
    y.view(torch.int16).fill_(FILL)
    ids_c = np_(ids)
    for n, (o, es) in enumerate(_shards(sh.experts, 8)):
        moe.moe_fused_fwd(inp["x"], gate[o:o + es], up[o:o + es], inp["w2"][o:o + es], ids, w,
                          expert_offset=o, num_global_experts=sh.experts, y_rows=y)
        if n == 0:
            # after the first shard only its own slots hold results
            untouched = (_bits(y) == FILL).all(axis=2)
            mine = (ids_c >= o) & (ids_c < o + es)
            assert (untouched == ~mine).all()
    assert not (_bits(y) == FILL).all(axis=2).any()
    out = moe.moe_combine(y, ids, w, sh.experts)
    assert (_bits(out) == _bits(full)).all()


@pytest.mark.parametrize("T", [33, 2048])
def test_bf16_ep_partial_out(w235, T):
    sh = W.QWEN3_235B_BF16
    inp = W.make_inputs(sh, T, seed=90 + T, device=DEV, weights=w235)
    (ids, w), (oi, ow) = route_both(inp)
    gate, up = W.packed_views(inp["w13"], sh.inter)
    o, es = 32, 32                                         # shard 1 of EP4
    part = moe.moe_fused_fwd(inp["x"], gate[o:o + es], up[o:o + es], inp["w2"][o:o + es], ids, w,
                             expert_offset=o, num_global_experts=sh.experts)
    foreign = (ids < o) | (ids >= o + es)
    masked = torch.where(foreign, torch.full_like(ids, -1), ids)
    ref = moe.moe_fused_fwd(inp["x"], gate, up, inp["w2"], masked, w)
    assert (_bits(part) == _bits(ref)).all()
    toks = sample_tokens(T, 6)
    om = np.where((oi < o) | (oi >= o + es), -1, oi).astype(np.int32)
    acc, _ = oracle_ffn_tokens(inp, om, ow, toks)
    got = bf16_to_f64(part[torch.from_numpy(toks).to(DEV)])
    r = rel_l2(got, acc)
    print(f"T={T} shard [{o}, {o + es}) rel_l2={r:.3e}")
    assert r <= 1e-2


@pytest.mark.parametrize("T", [64, 2048])
def test_mxfp4_ep4_rows_combine_to_unsharded(T):
    sh = W.QWEN35_397B_TP2_FP4_512
    g = torch.Generator(device=DEV).manual_seed(78)
    w13, w2 = W.draw_weights(sh, g, DEV)
    (gq, gs), (uq, us), (wq, wsc) = quantise_weights_gpu(w13, w2, sh.inter)
    inp = W.make_inputs(sh, T, seed=T, device=DEV, weights=(w13, w2))
    (ids, w), _ = route_both(inp)
    full = moe.moe_fused_fwd(inp["x"], gq, uq, wq, ids, w, gate_scale=gs, up_scale=us, w2_scale=wsc,
                             mode=moe.MODE_MXFP4)
    y = torch.empty((T, sh.top_k, sh.hidden), dtype=torch.bfloat16, device=DEV)
    y.view(torch.int16).fill_(FILL)
    for o, es in _shards(sh.experts, 4):
        moe.moe_fused_fwd(inp["x"], gq[o:o + es], uq[o:o + es], wq[o:o + es], ids, w,
                          gate_scale=gs[o:o + es], up_scale=us[o:o + es], w2_scale=wsc[o:o + es],
                          mode=moe.MODE_MXFP4, expert_offset=o, num_global_experts=sh.experts,
                          y_rows=y)
    out = moe.moe_combine(y, ids, w, sh.experts)
    assert (_bits(out) == _bits(full)).all()


def test_shard_with_no_local_slots():
    """A shard none of whose experts is picked writes no y row and, combining
    itself, an all-zero output."""
    sh = W.TINY_BF16
    inp = W.make_inputs(sh, 16, seed=5, device=DEV)
    ids = torch.randint(0, 4, (16, 2), dtype=torch.int32, device=DEV)      # experts 0..3 only
    w = torch.rand((16, 2), dtype=torch.float32, device=DEV)
    gate, up = W.packed_views(inp["w13"], sh.inter)
    y = torch.empty((16, 2, sh.hidden), dtype=torch.bfloat16, device=DEV)
    y.view(torch.int16).fill_(FILL)
    moe.moe_fused_fwd(inp["x"], gate[4:], up[4:], inp["w2"][4:], ids, w, expert_offset=4,
                      num_global_experts=8, y_rows=y)
    assert (_bits(y) == FILL).all()
    out = moe.moe_fused_fwd(inp["x"], gate[4:], up[4:], inp["w2"][4:], ids, w, expert_offset=4,
                            num_global_experts=8)
    assert (_bits(out) == 0).all()


def test_combine_strided_rows_and_ids():
    """moe_combine reads padded y rows and strided ids/weights, and equals the
    fused call's own combine."""
    sh = W.TINY_BF16
    T = 40
    inp = W.make_inputs(sh, T, seed=6, device=DEV, routing="replay")
    ids, w = inp["topk_ids"], inp["topk_weights"]
    gate, up = W.packed_views(inp["w13"], sh.inter)
    full = moe.moe_fused_fwd(inp["x"], gate, up, inp["w2"], ids, w)
    ypad = torch.zeros((T, sh.top_k, sh.hidden + 64), dtype=torch.bfloat16, device=DEV)
    y = ypad[:, :, :sh.hidden]
    moe.moe_fused_fwd(inp["x"], gate, up, inp["w2"], ids, w, y_rows=y)
    outt = torch.empty((sh.hidden, T), dtype=torch.bfloat16, device=DEV).t()
    moe.moe_combine(y, ids, w, sh.experts, out=outt)
    assert (_bits(outt) == _bits(full)).all()


def test_mxfp4_rows_out_at_one_token():
    """Per-slot rows at T = 1 (where the tuned choice folds the combine into
    gemm2) fall back to a kernel that writes rows; combined they equal the
    plain call bit for bit."""
    sh = W.QWEN35_397B_TP2_FP4_512
    g = torch.Generator(device=DEV).manual_seed(79)
    w13, w2 = W.draw_weights(sh, g, DEV)
    (gq, gs), (uq, us), (wq, wsc) = quantise_weights_gpu(w13, w2, sh.inter)
    inp = W.make_inputs(sh, 1, seed=1, device=DEV, weights=(w13, w2))
    (ids, w), _ = route_both(inp)
    kw = dict(gate_scale=gs, up_scale=us, w2_scale=wsc, mode=moe.MODE_MXFP4)
    full = moe.moe_fused_fwd(inp["x"], gq, uq, wq, ids, w, **kw)
    assert moe.moe_query_config(inp["x"], gq, uq, wq, ids, w, **kw)["gemm2_kernel"] == 16
    y = torch.zeros((1, sh.top_k, sh.hidden), dtype=torch.bfloat16, device=DEV)
    moe.moe_fused_fwd(inp["x"], gq, uq, wq, ids, w, y_rows=y, **kw)
    assert (_bits(moe.moe_combine(y, ids, w, sh.experts)) == _bits(full)).all()
