"""The fused forward captured in a HIP graph (through torch.cuda.CUDAGraph):
every replay equals the eager call bit for bit, with eager work on the same
buffers and synchronisations between the replays. The library allocates
nothing and records no memset nodes, so a call is capturable as is.

Cases: the Qwen3-235B-shaped bf16 layer at T = 512 (tiled GEMMs) and the TP2
MXFP4 shard at T = 64 (weight streams, multi-tile gemm2) and T = 2048 (two
block sizes, multi-launch align); the backward, the forward with the RMSNorm
pre-pass, and an expert-parallel shard followed by the home combine.
"""
import pytest
import torch

import mixture_experts_ffn_align_amd as moe
from mixture_experts_ffn_align_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _replays_match(call, x, x_other):
    """call(x) writes its output buffer; returns the eager result and checks
    four replays against it, with an eager call on other data in between."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            out = call(x)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = call(x)
    for r in range(4):
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager call"
        other = call(x_other).clone()            # eager work on the same buffers
        torch.cuda.synchronize()
        assert not torch.equal(other, eager)
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, eager)


def test_graph_bf16_t512():
    sh = W.QWEN3_235B_BF16
    g = torch.Generator(device=DEV).manual_seed(7)
    w13, w2 = W.draw_weights(sh, g, DEV)
    gate, up = W.packed_views(w13, sh.inter)
    inp = W.make_inputs(sh, 512, seed=3, device=DEV, weights=(w13, w2))
    ids, wts = moe.moe_topk_softmax(inp["logits"], sh.top_k)
    out = torch.empty(512, sh.hidden, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(moe.moe_fused_workspace_size(inp["x"], gate, up, w2, ids, wts), dtype=torch.uint8, device=DEV)
    xb = inp["x"].clone()

    def call(x):
        xb.copy_(x)
        return moe.moe_fused_fwd(xb, gate, up, w2, ids, wts, out=out, workspace=ws)

    _replays_match(call, inp["x"], inp["x"].flip(0).contiguous())


@pytest.mark.parametrize("T", [64, 2048])
def test_graph_mxfp4(T):
    sh = W.QWEN35_397B_TP2_FP4_512
    g = torch.Generator(device=DEV).manual_seed(11)
    w13, w2 = W.draw_weights(sh, g, DEV)
    gate, up = W.packed_views(w13, sh.inter)
    (gq, gs), (uq, us), (wq, wsc) = moe.moe_quant_mxfp4(gate), moe.moe_quant_mxfp4(up), moe.moe_quant_mxfp4(w2)
    del w13, w2, gate, up
    gx = torch.Generator(device=DEV).manual_seed(T)
    x = torch.randn(T, sh.hidden, generator=gx, device=DEV).to(torch.bfloat16)
    logits = torch.randn(T, sh.experts, generator=gx, device=DEV)
    ids, wts = moe.moe_topk_softmax(logits, sh.top_k)
    kw = dict(gate_scale=gs, up_scale=us, w2_scale=wsc, mode=moe.MODE_MXFP4)
    out = torch.empty(T, sh.hidden, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(moe.moe_fused_workspace_size(x, gq, uq, wq, ids, wts, **kw), dtype=torch.uint8, device=DEV)
    xb = x.clone()

    def call(xx):
        xb.copy_(xx)
        return moe.moe_fused_fwd(xb, gq, uq, wq, ids, wts, out=out, workspace=ws, **kw)

    _replays_match(call, x, (x * -0.5).contiguous())


def test_backward_norm_and_shard_replays_equal_eager():
    """The backward, the RMSNorm pre-pass inside the forward, and an
    expert-parallel shard with the home combine, each captured in a graph:
    every replay equals the eager result (the library records no memset and
    allocates nothing inside the call)."""
    sh = W.QWEN3_235B_BF16
    g = torch.Generator(device=DEV).manual_seed(8)
    w13, w2 = W.draw_weights(sh, g, DEV)
    gate, up = W.packed_views(w13, sh.inter)
    T = 256
    inp = W.make_inputs(sh, T, seed=9, device=DEV, weights=(w13, w2))
    ids, w = moe.moe_topk_softmax(inp["logits"], sh.routed_k)
    x = inp["x"]
    dout = torch.randn(T, sh.hidden, generator=torch.Generator(device=DEV).manual_seed(2),
                       device=DEV).to(torch.bfloat16)
    nw = torch.rand(sh.hidden, generator=torch.Generator(device=DEV).manual_seed(3), device=DEV)

    grads = [torch.empty_like(x), torch.empty((sh.experts, sh.inter, sh.hidden), device=DEV),
             torch.empty((sh.experts, sh.inter, sh.hidden), device=DEV),
             torch.empty((sh.experts, sh.hidden, sh.inter), device=DEV),
             torch.empty((T, sh.top_k), device=DEV)]
    ws_b = torch.empty(moe.moe_fused_bwd_workspace_size(x, gate, up, w2, ids, w, dout), dtype=torch.uint8,
                       device=DEV)

    def bwd():
        moe.moe_fused_bwd(x, gate, up, w2, ids, w, dout, dx=grads[0], dgate=grads[1], dup=grads[2],
                          dw2=grads[3], dtopk_weights=grads[4], workspace=ws_b)
        return grads

    out_n = torch.empty_like(x)
    ws_n = torch.empty(moe.moe_fused_workspace_size(x, gate, up, w2, ids, w, norm_weight=nw), dtype=torch.uint8,
                       device=DEV)

    def fwd_norm():
        moe.moe_fused_fwd(x, gate, up, w2, ids, w, out=out_n, workspace=ws_n, norm_weight=nw)
        return [out_n]

    es = sh.experts // 4
    y = torch.zeros((T, sh.top_k, sh.hidden), dtype=torch.bfloat16, device=DEV)
    out_c = torch.empty_like(x)
    ws_s = torch.empty(moe.moe_fused_workspace_size(x, gate[es:2 * es], up[es:2 * es], w2[es:2 * es], ids, w,
                                                    expert_offset=es, num_global_experts=sh.experts, y_rows=y),
                       dtype=torch.uint8, device=DEV)

    def shard():
        moe.moe_fused_fwd(x, gate[es:2 * es], up[es:2 * es], w2[es:2 * es], ids, w, workspace=ws_s,
                          expert_offset=es, num_global_experts=sh.experts, y_rows=y)
        moe.moe_combine(y, ids, w, sh.experts, out=out_c)
        return [y, out_c]

    for call in (bwd, fwd_norm, shard):
        eager = [t.clone() for t in call()]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            outs = call()
        for r in range(3):
            for t in outs:
                t.fill_(0)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for a, b in zip(outs, eager):
                assert torch.equal(a, b), (call.__name__, r)
