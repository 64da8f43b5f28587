"""moe_fused_fwd_noalloc: the fused forward on the library's built-in device
scratch (for callers that cannot allocate) against moe_fused_fwd with a
caller workspace, bit for bit, through the C ABI: two calls in a row, the
second with fewer tokens (the scratch keeps the first call's contents), in
bf16 and MXFP4, the few-token and the aligned paths; a call that needs more
than the scratch fails before any launch; and a graph that captures it
replays to the same bits."""
import pytest
import torch

import mixture_experts_ffn_align_amd as moe
from mixture_experts_ffn_align_amd import _abi
from mixture_experts_ffn_align_amd import workloads as W
from harness import quantise_weights_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"
LIMIT = 64 << 20


def _pair(args, kw, T_cut=None):
    ws = torch.empty(moe.moe_fused_workspace_size(*args, **kw), dtype=torch.uint8, device=DEV)
    assert ws.numel() <= LIMIT
    want = moe.moe_fused_fwd(*args, workspace=ws, **kw).clone()
    out = torch.full_like(want, float("nan"))
    got = moe.moe_fused_fwd_noalloc(*args, out=out, **kw)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(got, want)


def _slice(args, T):
    x, gate, up, w2, ids, w = args
    return (x[:T], gate, up, w2, ids[:T], w[:T])


@pytest.mark.parametrize("T1,T2", [(512, 100), (4, 1)])
def test_bf16_two_calls_second_smaller(T1, T2):
    sh = W.QWEN3_235B_BF16
    g = torch.Generator(device=DEV).manual_seed(3)
    w13, w2 = W.draw_weights(sh, g, DEV)
    inp = W.make_inputs(sh, T1, seed=T1, device=DEV, weights=(w13, w2))
    ids, w = moe.moe_topk_softmax(inp["logits"], sh.routed_k)
    gate, up = W.packed_views(w13, sh.inter)
    args = (inp["x"], gate, up, w2, ids, w)
    _pair(args, {})
    _pair(_slice(args, T2), {})
    # transposed activation and the RMSNorm pre-pass use more scratch segments
    xt = inp["x"].t().contiguous().t()
    nw = torch.rand(sh.hidden, generator=torch.Generator(device=DEV).manual_seed(1), device=DEV)
    _pair((xt[:T2],) + _slice(args, T2)[1:], dict(norm_weight=nw))


@pytest.mark.parametrize("T1,T2", [(64, 5), (512, 300)])
def test_mxfp4_two_calls_second_smaller(T1, T2):
    sh = W.QWEN35_397B_TP2_FP4_513
    g = torch.Generator(device=DEV).manual_seed(4)
    w13, w2 = W.draw_weights(sh, g, DEV)
    (gq, gs), (uq, us), (wq, wsc) = quantise_weights_gpu(w13, w2, sh.inter)
    del w13, w2
    inp_x = torch.randn(T1, sh.hidden, generator=g, device=DEV).to(torch.bfloat16)
    logits = torch.randn(T1, sh.routed_experts, generator=g, device=DEV)
    ids, w = moe.moe_topk_softmax(logits, sh.routed_k, shared_id=sh.shared_expert, shared_w=1.0)
    kw = dict(gate_scale=gs, up_scale=us, w2_scale=wsc, mode=moe.MODE_MXFP4)
    args = (inp_x, gq, uq, wq, ids, w)
    _pair(args, kw)
    _pair(_slice(args, T2), kw)


def test_too_large_fails_before_launch():
    sh = W.QWEN3_235B_BF16
    T = 4096
    x = torch.zeros(T, sh.hidden, dtype=torch.bfloat16, device=DEV)
    gate = torch.zeros(sh.experts, sh.inter, sh.hidden, dtype=torch.bfloat16, device=DEV)
    w2 = torch.zeros(sh.experts, sh.hidden, sh.inter, dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros(T, sh.top_k, dtype=torch.int32, device=DEV)
    w = torch.zeros(T, sh.top_k, device=DEV)
    assert moe.moe_fused_workspace_size(x, gate, gate, w2, ids, w) > LIMIT
    out = torch.full((T, sh.hidden), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_fused_fwd_noalloc(x, gate, gate, w2, ids, w, out=out)
    assert ei.value.status == -5 and "scratch" in ei.value.detail
    torch.cuda.synchronize()
    assert (out == 7.0).all()


def test_graph_capture_replays():
    sh = W.TINY_BF16
    inp = W.make_inputs(sh, 48, seed=8, device=DEV)
    ids, w = moe.moe_topk_softmax(inp["logits"], sh.routed_k)
    gate, up = W.packed_views(inp["w13"], sh.inter)
    args = (inp["x"], gate, up, inp["w2"], ids, w)
    want = moe.moe_fused_fwd(*args, workspace=torch.empty(moe.moe_fused_workspace_size(*args), dtype=torch.uint8,
                                                           device=DEV)).clone()
    out = torch.empty_like(want)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.moe_fused_fwd_noalloc(*args, out=out)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.moe_fused_fwd_noalloc(*args, out=out)
    for _ in range(3):
        out.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want)
        moe.moe_fused_fwd_noalloc(*args, out=torch.empty_like(out))   # eager calls between replays
        torch.cuda.synchronize()


def test_symbol_is_exported():
    assert hasattr(_abi.load(), "moe_fused_fwd_noalloc")
