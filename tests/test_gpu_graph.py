"""The fused forward captured in a HIP graph (through torch.cuda.CUDAGraph):
every replay equals the eager call bit for bit, with eager work on the same
buffers and synchronisations between the replays. The library allocates
nothing and records no memset nodes, so a call is capturable as is.

Cases: the Qwen3-235B-shaped bf16 layer at T = 512 (tiled GEMMs) and the TP2
MXFP4 shard at T = 64 (weight streams, multi-tile gemm2) and T = 2048 (two
block sizes, multi-launch align).
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
