"""GPU parity of the fused forward against the oracle, per workload:

* tiny bf16 (every token compared);
* Qwen3-235B-shaped bf16 at T = 512 (sampled tokens);
* the same weights passed as packed w13 views with router-replay id slices
  (token stride 46*8), bit-identical to contiguous copies, T = 4096 and 16384;
* Zipf-skewed routing with an activation stored transposed (last-dim stride
  T), T = 1, 7, 333, 4099, bit-identical to a contiguous activation;
* Qwen3.5-397B TP2 MXFP4 shard, 512/10 and 513/11, token buckets 1 ... 32768.

Tolerances: bf16 rel-L2 <= 1e-2 and errRatio <= 0.05; MXFP4 rel-L2 <= 2e-2
and errRatio <= 0.05, errRatio being the fraction of elements with
|gpu - ref| > 1e-2 * |ref| + 1e-2 * rms(ref). Router ids and weights and the
align are bit-exact (test_gpu_steps). From 4096 tokens up the oracle sees at
least 256 tokens per case, among them the token of every expert's last
assignment, which sits in that expert's ragged last sorted block.
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_align_amd as moe
from mixture_experts_ffn_align_amd import workloads as W
from harness import (assert_routing_equal, bf16_to_f64, err_ratio, np_, oracle_ffn_tokens,
                     oracle_quant_experts, quantise_weights_gpu, rel_l2, route_both,
                     sample_tokens, tail_tokens)

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16_TOL = 1e-2
FP4_TOL = 2e-2
FP4_ERR_RATIO = 0.05


def _fused_bf16(inp, ids, w, *, gate=None, up=None, x=None, out=None, force_config=-1):
    sh = inp["shape"]
    if gate is None:
        gate, up = W.packed_views(inp["w13"], sh.inter)
    return moe.moe_fused_fwd(inp["x"] if x is None else x, gate, up, inp["w2"], ids, w, out=out,
                             force_config=force_config)


def _check_bf16(inp, out, oi, ow, toks):
    acc, _ = oracle_ffn_tokens(inp, oi, ow, toks)
    got = bf16_to_f64(out[torch.from_numpy(toks).to(out.device)])
    r, er = rel_l2(got, acc), err_ratio(got, acc)
    print(f"{len(toks)} tokens: rel_l2={r:.3e} err_ratio={er:.3e}")
    assert np.isfinite(got).all()
    assert r <= BF16_TOL and er <= FP4_ERR_RATIO
    return r


@pytest.fixture(scope="module")
def w235():
    g = torch.Generator(device=DEV).manual_seed(1234)
    return W.draw_weights(W.QWEN3_235B_BF16, g, DEV)


@pytest.mark.parametrize("T", [64, 1, 7, 100])
def test_tiny_bf16_every_token(T):
    inp = W.make_inputs(W.TINY_BF16, T, seed=T, device=DEV)
    gpu, orc = route_both(inp)
    assert_routing_equal(gpu, orc)
    out = _fused_bf16(inp, *gpu)
    r = _check_bf16(inp, out, *orc, np.arange(T))
    assert r < 3e-3          # only bf16 rounding of h, y and out separates the two


def test_tiny_bf16_tile_configs():
    """Configs that split K the same way give identical bits; all are within tolerance."""
    inp = W.make_inputs(W.TINY_BF16, 64, seed=9, device=DEV)
    gpu, orc = route_both(inp)
    outs = {}
    info = moe.moe_query_config(inp["x"], *W.packed_views(inp["w13"], 128), inp["w2"], *gpu)
    for c in range(info["num_configs"]):
        try:
            outs[c] = _fused_bf16(inp, *gpu, force_config=c).clone()
        except moe.MoEError as err:          # a config this shape cannot use
            assert err.status == -6, err
    assert len(outs) >= 6
    groups = {}
    for c in outs:
        _check_bf16(inp, outs[c], *orc, np.arange(64))
        q = moe.moe_query_config(inp["x"], *W.packed_views(inp["w13"], 128), inp["w2"], *gpu,
                                 force_config=c)
        groups.setdefault((q["gemm1_split_k"], q["gemm2_split_k"]), []).append(c)
    # the K split fixes the summation order; block_m does not change any bit
    for cs in groups.values():
        for c in cs[1:]:
            assert torch.equal(outs[c], outs[cs[0]]), f"config {c} differs from {cs[0]}"
    assert any(len(cs) > 1 for cs in groups.values())


def test_qwen3_235b_bf16_t512(w235):
    inp = W.make_inputs(W.QWEN3_235B_BF16, 512, seed=0, device=DEV, weights=w235)
    gpu, orc = route_both(inp)
    assert_routing_equal(gpu, orc)
    out = _fused_bf16(inp, *gpu)
    assert torch.isfinite(out.float()).all()
    _check_bf16(inp, out, *orc, tail_tokens(orc[0], 128, 64))


@pytest.mark.parametrize("T", [4096, 16384])
def test_packed_views_and_replay_slices_bit_identical(w235, T):
    inp = W.make_inputs(W.QWEN3_235B_BF16, T, seed=0, device=DEV, routing="replay", weights=w235)
    gate, up = W.packed_views(inp["w13"], 1536)
    ids, w = inp["topk_ids"], inp["topk_weights"]
    assert gate.stride(0) == 2 * 1536 * 4096 and ids.stride(0) == 46 * 8
    cfg_s = moe.moe_query_config(inp["x"], gate, up, inp["w2"], ids, w)
    cfg_c = moe.moe_query_config(inp["x"], gate.contiguous(), up.contiguous(), inp["w2"],
                                 ids.contiguous(), w.contiguous())
    assert cfg_s == cfg_c
    out_s = _fused_bf16(inp, ids, w, gate=gate, up=up).clone()
    out_c = _fused_bf16(inp, ids.contiguous(), w.contiguous(), gate=gate.contiguous(),
                        up=up.contiguous()).clone()
    assert torch.equal(out_s, out_c)
    _check_bf16(inp, out_s, np_(ids), np_(w), tail_tokens(np_(ids), 128, 256))


@pytest.mark.parametrize("T", [1, 7, 333, 4099])
def test_zipf_skew_transposed_x_bit_identical(w235, T):
    inp = W.make_inputs(W.QWEN3_235B_BF16, T, seed=0, device=DEV, logits_kind="zipf",
                        x_layout="transposed", weights=w235)
    assert inp["x"].stride() == (1, T)
    gpu, orc = route_both(inp)
    assert_routing_equal(gpu, orc)
    out_t = _fused_bf16(inp, *gpu).clone()
    out_c = _fused_bf16(inp, *gpu, x=inp["x"].contiguous()).clone()
    assert torch.equal(out_t, out_c)
    if T >= 333:
        used = np.unique(orc[0])
        assert used.size < 128          # the skew leaves experts without tokens
    _check_bf16(inp, out_t, *orc, tail_tokens(orc[0], 128, 256 if T >= 4096 else 6))


@pytest.fixture(scope="module")
def fp4_weights():
    cache = {}

    def get(shape):
        if shape.name not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            g = torch.Generator(device=DEV).manual_seed(77)
            w13, w2 = W.draw_weights(shape, g, DEV)
            q = quantise_weights_gpu(w13, w2, shape.inter)
            cache[shape.name] = (w13, w2, q, {})
        return cache[shape.name][:3]
    get.oracle_codes = lambda shape, used: _oracle_codes(cache[shape.name], shape, used)
    return get


def _oracle_codes(entry, shape, used):
    """The oracle's own MXFP4 codes of the listed experts, quantised once per
    expert and kept for the module (the large buckets touch all 512)."""
    w13, w2, _, memo = entry
    missing = [e for e in used if e not in memo]
    if missing:
        memo.update(oracle_quant_experts(w13, w2, shape.inter, missing))
    return {e: memo[e] for e in used}


@pytest.mark.parametrize("T", [1, 2, 16, 64, 512, 4096, 8192, 16384, 32768])
@pytest.mark.parametrize("shape", [W.QWEN35_397B_TP2_FP4_512, W.QWEN35_397B_TP2_FP4_513],
                         ids=["512x10", "513x11"])
def test_mxfp4_tp2_shard(fp4_weights, shape, T):
    w13, w2, ((gq, gs), (uq, us), (wq, wsc)) = fp4_weights(shape)
    inp = W.make_inputs(shape, T, seed=T, device=DEV, weights=(w13, w2))
    gpu, orc = route_both(inp)
    assert_routing_equal(gpu, orc)
    out = moe.moe_fused_fwd(inp["x"], gq, uq, wq, *gpu, gate_scale=gs, up_scale=us, w2_scale=wsc,
                            mode=moe.MODE_MXFP4)
    oi, ow = orc
    toks = tail_tokens(oi, shape.experts, 256) if T >= 4096 else sample_tokens(T, 4)
    used = sorted({int(e) for e in oi[toks].ravel()})
    mx = fp4_weights.oracle_codes(shape, used)
    for e in used[:3]:                      # GPU weight codes equal the oracle's
        (ocg, osg), _, (ocd, osd) = mx[e]
        assert (np_(gq[e]) == ocg).all() and (np_(gs[e]) == osg).all()
        assert (np_(wq[e]) == ocd).all() and (np_(wsc[e]) == osd).all()
    acc, _ = oracle_ffn_tokens(inp, oi, ow, toks, mx=mx)
    got = bf16_to_f64(out[torch.from_numpy(toks).to(DEV)])
    r, er = rel_l2(got, acc), err_ratio(got, acc)
    print(f"T={T} {len(toks)} tokens rel_l2={r:.3e} err_ratio={er:.3e}")
    assert np.isfinite(got).all()
    assert r <= FP4_TOL and er <= FP4_ERR_RATIO


def _configs_by_family(query):
    """config index of each GEMM kernel family the library lists"""
    n = query(-1)["num_configs"]
    fam = {}
    for c in range(n):
        try:
            q = query(c)
        except moe.MoEError as err:
            assert err.status == -6, err
            continue
        fam.setdefault((q["gemm1_kernel"], q["gemm1_split_k"], q["gemm2_split_k"]), []).append(c)
    return fam


def test_tiled_and_streaming_gemms_same_bits_bf16(w235):
    """Both GEMM families sum K in the same order: identical outputs."""
    inp = W.make_inputs(W.QWEN3_235B_BF16, 4096, seed=3, device=DEV, weights=w235)
    gpu, orc = route_both(inp)
    gate, up = W.packed_views(inp["w13"], 1536)
    fam = _configs_by_family(lambda c: moe.moe_query_config(inp["x"], gate, up, inp["w2"], *gpu,
                                                            force_config=c))
    assert len(fam[(3, 1, 1)]) >= 6          # every tile shape (128 x 256 with two gemm2 choices)
    assert moe.moe_query_config(inp["x"], gate, up, inp["w2"], *gpu)["gemm1_kernel"] == 3
    out_s = _fused_bf16(inp, *gpu, force_config=fam[(1, 1, 1)][-1]).clone()
    for c in fam[(3, 1, 1)]:
        out_t = _fused_bf16(inp, *gpu, force_config=c)
        assert torch.equal(out_t, out_s), f"config {c}"
    _check_bf16(inp, out_s, *orc, tail_tokens(orc[0], 128, 128))


@pytest.mark.parametrize("T", [64, 2048])
def test_tiled_and_streaming_gemms_same_bits_mxfp4(fp4_weights, T):
    shape = W.QWEN35_397B_TP2_FP4_513
    w13, w2, ((gq, gs), (uq, us), (wq, wsc)) = fp4_weights(shape)
    inp = W.make_inputs(shape, T, seed=5, device=DEV, weights=(w13, w2))
    gpu, orc = route_both(inp)

    def run(c):
        return moe.moe_fused_fwd(inp["x"], gq, uq, wq, *gpu, gate_scale=gs, up_scale=us, w2_scale=wsc,
                                 mode=moe.MODE_MXFP4, force_config=c).clone()

    def query(c):
        return moe.moe_query_config(inp["x"], gq, uq, wq, *gpu, gate_scale=gs, up_scale=us,
                                    w2_scale=wsc, mode=moe.MODE_MXFP4, force_config=c)

    fam = _configs_by_family(query)
    assert len(fam[(13, 1, 1)]) >= 5          # every MXFP4 tile shape, and mixed gemm2 choices
    assert len(fam[(19, 1, 1)]) >= 8          # the persistent gemm1 with 4 and 8 waves
    out_t = run(fam[(13, 1, 1)][0])
    for c in fam[(13, 1, 1)][1:] + fam[(11, 1, 1)] + fam[(19, 1, 1)]:
        assert torch.equal(run(c), out_t), f"config {c}"
    toks = sample_tokens(T, 4)
    oi, ow = orc
    used = sorted({int(e) for e in oi[toks].ravel()})
    acc, _ = oracle_ffn_tokens(inp, oi, ow, toks, mx=oracle_quant_experts(w13, w2, shape.inter, used))
    got = bf16_to_f64(out_t[torch.from_numpy(toks).to(DEV)])
    assert rel_l2(got, acc) <= FP4_TOL and err_ratio(got, acc) <= FP4_ERR_RATIO


def test_nan_canaries_in_unread_memory():
    """Unused half of the packed w13, padding columns of x and the other
    layers of the routing tensors hold NaN / out-of-range values; any read of
    them would show in the output. Writes stay inside out's view."""
    sh = W.TINY_BF16
    inp = W.make_inputs(sh, 40, seed=5, device=DEV)
    gpu, orc = route_both(inp)
    ref = _fused_bf16(inp, *gpu, gate=inp["w13"][:, :128].contiguous(),
                      up=inp["w13"][:, 128:].contiguous()).clone()
    w13 = inp["w13"].clone()
    w13[:, 128:, :] = float("nan")
    gate = w13[:, :128, :]
    up = inp["w13"][:, 128:, :].contiguous()
    xbuf = torch.full((40, 256 + 64), float("nan"), dtype=torch.bfloat16, device=DEV)
    xbuf[:, 32:288] = inp["x"]
    x = xbuf[:, 32:288]
    ids_all = torch.full((1, 40, 5, 2), 999, dtype=torch.int32, device=DEV)
    w_all = torch.full((1, 40, 5, 2), float("nan"), device=DEV)
    ids_all[0, :, 3, :] = gpu[0]
    w_all[0, :, 3, :] = gpu[1]
    obuf = torch.full((40, 3, 256), float("nan"), dtype=torch.bfloat16, device=DEV)
    out = obuf[:, 1, :]
    moe.moe_fused_fwd(x, gate, up, inp["w2"], ids_all[0, :, 3, :], w_all[0, :, 3, :], out=out)
    assert torch.equal(out, ref)
    assert torch.isnan(obuf[:, 0].float()).all() and torch.isnan(obuf[:, 2].float()).all()


def test_run_twice_bit_identical_and_zero_weight_slot(w235):
    inp = W.make_inputs(W.QWEN3_235B_BF16, 333, seed=3, device=DEV, weights=w235)
    ids, w = route_both(inp)[0]
    a = _fused_bf16(inp, ids, w).clone()
    b = _fused_bf16(inp, ids, w).clone()
    assert torch.equal(a, b)
    w0 = w.clone()
    w0[:, 3] = 0.0
    ids_drop = ids.clone()
    ids_drop[:, 3] = -1
    c = _fused_bf16(inp, ids, w0).clone()
    d = _fused_bf16(inp, ids_drop, w0).clone()
    assert torch.equal(c, d)
    # scaling every weight by 2 scales the output by exactly 2
    e2 = _fused_bf16(inp, ids, 2 * w).clone()
    assert torch.equal(e2.float(), 2 * a.float())


def test_empty_batch_and_graph_capture():
    sh = W.TINY_BF16
    inp = W.make_inputs(sh, 48, seed=8, device=DEV)
    ids, w = route_both(inp)[0]
    empty = moe.moe_fused_fwd(inp["x"][:0], *W.packed_views(inp["w13"], 128), inp["w2"], ids[:0], w[:0])
    assert empty.shape == (0, 256)
    gate, up = W.packed_views(inp["w13"], 128)
    nbytes = moe.moe_fused_workspace_size(inp["x"], gate, up, inp["w2"], ids, w)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    out = torch.empty(48, 256, dtype=torch.bfloat16, device=DEV)
    eager = moe.moe_fused_fwd(inp["x"], gate, up, inp["w2"], ids, w, workspace=ws).clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.moe_fused_fwd(inp["x"], gate, up, inp["w2"], ids, w, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.moe_fused_fwd(inp["x"], gate, up, inp["w2"], ids, w, out=out, workspace=ws)
    for _ in range(3):
        out.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        _ = moe.moe_fused_fwd(inp["x"], gate, up, inp["w2"], ids, w, workspace=ws)


@pytest.mark.parametrize("T", [1, 8, 32])
def test_mxfp4_gemm1_per_slot_same_bits(fp4_weights, T):
    """MXFP4 gemm1 per slot without the align (kernel family 17, K split 4)
    gives the same bits as the register weight stream with the same split,
    for contiguous and transposed activations and with the RMSNorm pre-pass;
    and matches the oracle."""
    shape = W.QWEN35_397B_TP2_FP4_512
    w13, w2, ((gq, gs), (uq, us), (wq, wsc)) = fp4_weights(shape)
    inp = W.make_inputs(shape, T, seed=70 + T, device=DEV, weights=(w13, w2))
    gpu, orc = route_both(inp)
    kw = dict(gate_scale=gs, up_scale=us, w2_scale=wsc, mode=moe.MODE_MXFP4)

    def query(c):
        return moe.moe_query_config(inp["x"], gq, uq, wq, *gpu, force_config=c, **kw)
    fam = _configs_by_family(query)
    small = fam[(17, 4, 1)]
    stream = fam[(11, 4, 1)]
    nw = torch.rand(shape.hidden, generator=torch.Generator(device=DEV).manual_seed(2), device=DEV)
    # a bf16 norm weight with element stride 3 (the per-slot gemm1 folds the
    # norm in; the stream configs run the separate pass)
    nwb = torch.rand(3 * shape.hidden, generator=torch.Generator(device=DEV).manual_seed(4),
                     device=DEV).to(torch.bfloat16)[::3]
    xt = inp["x"].t().contiguous().t()
    for x, extra in ((inp["x"], {}), (xt, {}), (inp["x"], dict(norm_weight=nw)),
                     (xt, dict(norm_weight=nwb, norm_eps=1e-3))):
        ref = moe.moe_fused_fwd(x, gq, uq, wq, *gpu, force_config=stream[0], **extra, **kw).clone()
        for c in small + stream[1:]:
            got = moe.moe_fused_fwd(x, gq, uq, wq, *gpu, force_config=c, **extra, **kw)
            assert torch.equal(got, ref), f"config {c}"
    out = moe.moe_fused_fwd(inp["x"], gq, uq, wq, *gpu, force_config=small[0], **kw)
    toks = sample_tokens(T, 4)
    oi, ow = orc
    used = sorted({int(e) for e in oi[toks].ravel()})
    acc, _ = oracle_ffn_tokens(inp, oi, ow, toks, mx=oracle_quant_experts(w13, w2, shape.inter, used))
    got = bf16_to_f64(out[torch.from_numpy(toks).to(DEV)])
    assert rel_l2(got, acc) <= FP4_TOL and err_ratio(got, acc) <= FP4_ERR_RATIO


@pytest.mark.parametrize("T", [1, 5, 16])
def test_bf16_per_slot_and_fused_gemm2_same_bits(w235, T):
    """bf16 gemm1 per slot without the align (family 7) and gemm2 with the
    combine folded in (family 6), both with a 4-way K split, give the same
    bits as the weight streams with that split followed by the separate
    combine, for contiguous and transposed activations, packed w13 views and
    the RMSNorm pre-pass; and match the oracle."""
    sh = W.QWEN3_235B_BF16
    inp = W.make_inputs(sh, T, seed=80 + T, device=DEV, weights=w235)
    gpu, orc = route_both(inp)
    gate, up = W.packed_views(inp["w13"], sh.inter)

    def query(c):
        return moe.moe_query_config(inp["x"], gate, up, inp["w2"], *gpu, force_config=c)
    n = query(-1)["num_configs"]
    kinds = {}
    for c in range(n):
        try:
            q = query(c)
        except moe.MoEError as err:
            assert err.status == -6, err
            continue
        if q["gemm1_split_k"] == 4 and q["gemm2_split_k"] == 4:
            kinds.setdefault((q["gemm1_kernel"], q["gemm2_kernel"]), []).append(c)
    assert (1, 2) in kinds and (1, 6) in kinds and (7, 6) in kinds, kinds
    ref_cfg = kinds[(1, 2)][0]
    others = [c for key, cs in kinds.items() for c in cs if c != ref_cfg]
    nw = torch.rand(sh.hidden, generator=torch.Generator(device=DEV).manual_seed(3), device=DEV)
    nwb = torch.rand(3 * sh.hidden, generator=torch.Generator(device=DEV).manual_seed(5),
                     device=DEV).to(torch.bfloat16)[::3]
    xt = inp["x"].t().contiguous().t()
    gc, uc = gate.contiguous(), up.contiguous()
    for x, g_, u_, extra in ((inp["x"], gate, up, {}), (xt, gc, uc, {}), (inp["x"], gate, up, dict(norm_weight=nw)),
                             (xt, gate, up, dict(norm_weight=nwb, norm_eps=1e-3))):
        ref = moe.moe_fused_fwd(x, g_, u_, inp["w2"], *gpu, force_config=ref_cfg, **extra).clone()
        for c in others:
            got = moe.moe_fused_fwd(x, g_, u_, inp["w2"], *gpu, force_config=c, **extra)
            assert torch.equal(got, ref), f"config {c}"
    out = moe.moe_fused_fwd(inp["x"], gate, up, inp["w2"], *gpu, force_config=kinds[(7, 6)][0])
    toks = sample_tokens(T, 4)
    oi, ow = orc
    acc, _ = oracle_ffn_tokens(inp, oi, ow, toks)
    got = bf16_to_f64(out[torch.from_numpy(toks).to(DEV)])
    assert rel_l2(got, acc) <= 1e-2


def test_few_token_kernels_reject_unsupported_shapes(w235):
    """The per-slot gemm1 needs H a multiple of 2048 and the fused bf16 gemm2
    I a multiple of 256 up to 1536; the configs that use them on the
    Qwen3-235B shape, forced on the tiny layer (H=256, I=128), fail with
    MOE_ERR_UNSUPPORTED, and the tiny layer's default never picks them."""
    big = W.make_inputs(W.QWEN3_235B_BF16, 1, seed=9, device=DEV, weights=w235, routing="replay")
    bg, bu = W.packed_views(big["w13"], 1536)
    n = moe.moe_query_config(big["x"], bg, bu, big["w2"], big["topk_ids"], big["topk_weights"])["num_configs"]
    few = []
    for c in range(n):
        try:
            q = moe.moe_query_config(big["x"], bg, bu, big["w2"], big["topk_ids"], big["topk_weights"],
                                     force_config=c)
        except moe.MoEError:
            continue
        if q["gemm1_kernel"] == 7 or q["gemm2_kernel"] == 6:
            few.append(c)
    assert few
    sh = W.TINY_BF16
    inp = W.make_inputs(sh, 3, seed=9, device=DEV, routing="replay")
    gate, up = W.packed_views(inp["w13"], sh.inter)
    ids, w = inp["topk_ids"], inp["topk_weights"]
    for c in few:
        with pytest.raises(moe.MoEError) as ei:
            moe.moe_fused_fwd(inp["x"], gate, up, inp["w2"], ids, w, force_config=c)
        assert ei.value.status == -6
    q = moe.moe_query_config(inp["x"], gate, up, inp["w2"], ids, w)
    assert q["gemm1_kernel"] in (1, 3) and q["gemm2_kernel"] in (2, 4)


@pytest.mark.parametrize("k", [33, 40])
def test_mxfp4_fused_gemm2_many_slots(k):
    """More than 32 slots per token take the fused gemm2's multi-round
    variant (16 waves, two slots each per round): bit-identical to gemm2 on
    the multi-tile stream followed by the separate combine, with the same K
    splits, including an invalid id and a zero weight."""
    T, H, I, E = 5, 2048, 512, 48
    g = torch.Generator(device=DEV).manual_seed(k)
    w13 = (torch.randn(E, 2 * I, H, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    w2 = (torch.randn(E, H, I, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    gate, up = W.packed_views(w13, I)
    (gq, gs), (uq, us), (wq, wsc) = moe.moe_quant_mxfp4(gate), moe.moe_quant_mxfp4(up), moe.moe_quant_mxfp4(w2)
    x = torch.randn(T, H, generator=g, device=DEV).to(torch.bfloat16)
    ids = torch.stack([torch.randperm(E, generator=g, device=DEV)[:k] for _ in range(T)]).to(torch.int32)
    ids[1, 5] = -1
    w = torch.rand(T, k, generator=g, device=DEV)
    w[2, 7] = 0.0
    kw = dict(gate_scale=gs, up_scale=us, w2_scale=wsc, mode=moe.MODE_MXFP4)
    n = moe.moe_query_config(x, gq, uq, wq, ids, w, **kw)["num_configs"]
    fused, plain = [], []
    for c in range(n):
        try:
            q = moe.moe_query_config(x, gq, uq, wq, ids, w, force_config=c, **kw)
        except moe.MoEError:
            continue
        if q["gemm1_kernel"] in (11, 17) and q["gemm1_split_k"] == 4 and q["gemm2_split_k"] == 1:
            (fused if q["gemm2_kernel"] == 16 else plain).append(c)
    assert fused and plain, (fused, plain)
    ref = moe.moe_fused_fwd(x, gq, uq, wq, ids, w, force_config=plain[0], **kw).clone()
    for c in fused:
        assert torch.equal(moe.moe_fused_fwd(x, gq, uq, wq, ids, w, force_config=c, **kw), ref), f"config {c}"


def _few_token_same_bits(mode, H, I, E, k, T, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    w13 = (torch.randn(E, 2 * I, H, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    w2 = (torch.randn(E, H, I, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    gate, up = W.packed_views(w13, I)
    kw = {}
    if mode == moe.MODE_MXFP4:
        (gate, gs), (up, us), (w2, wsc) = moe.moe_quant_mxfp4(gate), moe.moe_quant_mxfp4(up), moe.moe_quant_mxfp4(w2)
        kw = dict(gate_scale=gs, up_scale=us, w2_scale=wsc, mode=mode)
    x = torch.randn(T, H, generator=g, device=DEV).to(torch.bfloat16)
    ids = torch.stack([torch.randperm(E, generator=g, device=DEV)[:k] for _ in range(T)]).to(torch.int32)
    w = torch.rand(T, k, generator=g, device=DEV)
    per_slot, fused_only, plain = (7, 6, 4) if mode == moe.MODE_BF16 else (17, 16, 1)
    n = moe.moe_query_config(x, gate, up, w2, ids, w, **kw)["num_configs"]
    want = {}
    for c in range(n):
        try:
            q = moe.moe_query_config(x, gate, up, w2, ids, w, force_config=c, **kw)
        except moe.MoEError:
            continue
        if q["gemm1_split_k"] == 4 and q["gemm2_split_k"] == plain:
            want.setdefault((q["gemm1_kernel"], q["gemm2_kernel"]), []).append(c)
    keys = sorted(want)
    assert any(key[0] == per_slot for key in keys) and any(key[1] == fused_only for key in keys), keys
    # the weight streams with the same split as reference where K allows
    # that split; else the per-slot kernels against gemm1 on the stream
    stream = [key for key in keys if key[0] != per_slot and key[1] != fused_only] or \
        [key for key in keys if key[0] != per_slot]
    assert stream, keys
    # also with the RMSNorm, which the per-slot gemm1 folds in (the others
    # run the separate pass): an fp32 weight, or a bf16 one with stride 2
    nw = torch.rand(2 * H, generator=g, device=DEV)
    nw = nw[:H] if seed % 2 else nw.to(torch.bfloat16)[::2]
    for extra in ({}, dict(norm_weight=nw)):
        ref = moe.moe_fused_fwd(x, gate, up, w2, ids, w, force_config=want[stream[0]][0], **extra, **kw).clone()
        for key in keys:
            for c in want[key]:
                got = moe.moe_fused_fwd(x, gate, up, w2, ids, w, force_config=c, **extra, **kw)
                assert torch.equal(got, ref), (key, c, bool(extra))


@pytest.mark.parametrize("H,I,k", [(2048, 512, 6), (6144, 1024, 10), (8192, 768, 3)])
def test_bf16_few_token_kernels_other_shapes(H, I, k):
    """The bf16 per-slot gemm1 and fused gemm2 at other row lengths, widths
    and slot counts (every template instance of the row length): the same
    bits as the weight streams with a 4-way K split and the separate
    combine."""
    _few_token_same_bits(moe.MODE_BF16, H, I, 24, k, 3, seed=H + k)


@pytest.mark.parametrize("H,k", [(2048, 10), (6144, 7), (8192, 11)])
def test_mxfp4_few_token_kernels_other_shapes(H, k):
    """The MXFP4 per-slot gemm1 at other row lengths (every template instance)
    and slot counts: the same bits as the weight stream with a 4-way K split
    (at H = 8192 this caught the stream's scale staging overflowing its LDS
    rows)."""
    _few_token_same_bits(moe.MODE_MXFP4, H, 512, 24, k, 3, seed=H + k)


@pytest.mark.parametrize("T", [1, 5, 333, 4099, 9000])
def test_mxfp4_persistent_streams(fp4_weights, T):
    """The persistent weight streams (gemm1, gemm2 with K = 512, or both: one
    workgroup per compute unit walking its items, the weight ring running on
    across them) against the per-item weight stream: bit-identical h and y,
    so identical outputs, from fewer items than compute units (T = 1, 5) to
    more than a hundred items per workgroup (T = 9000); sampled tokens (the
    experts' tail blocks from T = 4099 on) against the oracle."""
    shape = W.QWEN35_397B_TP2_FP4_512 if T % 2 else W.QWEN35_397B_TP2_FP4_513
    w13, w2, ((gq, gs), (uq, us), (wq, wsc)) = fp4_weights(shape)
    inp = W.make_inputs(shape, T, seed=T + 11, device=DEV, weights=(w13, w2))
    gpu, orc = route_both(inp)
    kw = dict(gate_scale=gs, up_scale=us, w2_scale=wsc, mode=moe.MODE_MXFP4)
    n = moe.moe_query_config(inp["x"], gq, uq, wq, *gpu, **kw)["num_configs"]
    pers, plain = [], []
    for c in range(n):
        try:
            q = moe.moe_query_config(inp["x"], gq, uq, wq, *gpu, force_config=c, **kw)
        except moe.MoEError as err:
            assert err.status == -6, err
            continue
        if q["gemm1_split_k"] != 1 or q["gemm2_split_k"] != 1:
            continue
        (pers if q["gemm1_kernel"] == 19 or q["gemm2_kernel"] == 20 else plain).append(c)
    # 16-row blocks of gemm2 exceed 256 items per compute unit from about 6000 tokens
    assert len(pers) >= (14 if T < 6000 else 10)
    out_r = moe.moe_fused_fwd(inp["x"], gq, uq, wq, *gpu, force_config=plain[0], **kw).clone()
    for c in pers:
        out_p = moe.moe_fused_fwd(inp["x"], gq, uq, wq, *gpu, force_config=c, **kw)
        assert torch.equal(out_p, out_r), f"config {c}"
    oi, ow = orc
    toks = tail_tokens(oi, shape.experts, 64) if T >= 4096 else sample_tokens(T, 4)
    used = sorted({int(e) for e in oi[toks].ravel()})
    acc, _ = oracle_ffn_tokens(inp, oi, ow, toks, mx=fp4_weights.oracle_codes(shape, used))
    got = bf16_to_f64(out_r[torch.from_numpy(toks).to(DEV)])
    assert rel_l2(got, acc) <= FP4_TOL and err_ratio(got, acc) <= FP4_ERR_RATIO


def test_mxfp4_long_rows_every_config_against_oracle():
    """MXFP4 with H = 8192 (scale runs longer than a K split's LDS share):
    every configuration the library accepts matches the oracle."""
    import dataclasses
    sh = dataclasses.replace(W.QWEN35_397B_TP2_FP4_512, name="mxfp4_h8192_i512_e16_k4", hidden=8192, experts=16,
                             top_k=4, routed_experts=16, routed_k=4)
    g = torch.Generator(device=DEV).manual_seed(3)
    w13, w2 = W.draw_weights(sh, g, DEV)
    (gq, gs), (uq, us), (wq, wsc) = quantise_weights_gpu(w13, w2, sh.inter)
    T = 3
    inp = W.make_inputs(sh, T, seed=4, device=DEV, weights=(w13, w2), routing="replay")
    ids, w = inp["topk_ids"], inp["topk_weights"]
    kw = dict(gate_scale=gs, up_scale=us, w2_scale=wsc, mode=moe.MODE_MXFP4)
    oi, ow = np_(ids), np_(w)
    toks = np.arange(T)
    used = sorted({int(e) for e in oi.ravel()})
    acc, _ = oracle_ffn_tokens(inp, oi, ow, toks, mx=oracle_quant_experts(w13, w2, sh.inter, used))
    n = moe.moe_query_config(inp["x"], gq, uq, wq, ids, w, **kw)["num_configs"]
    ran = 0
    for c in range(n):
        try:
            moe.moe_query_config(inp["x"], gq, uq, wq, ids, w, force_config=c, **kw)
        except moe.MoEError:
            continue
        got = bf16_to_f64(moe.moe_fused_fwd(inp["x"], gq, uq, wq, ids, w, force_config=c, **kw))
        assert rel_l2(got, acc) <= FP4_TOL and err_ratio(got, acc) <= FP4_ERR_RATIO, c
        ran += 1
    assert ran >= 30


def test_bf16_oversized_call_in_token_chunks(w235):
    """90000 tokens on the bf16 Qwen3-235B-shaped layer run as chunks of
    32768 tokens with the whole call's configuration: every chunk's rows
    equal a call on those rows alone (bit for bit), and sampled tokens,
    including the experts' ragged tail blocks, match the oracle."""
    sh = W.QWEN3_235B_BF16
    T = 90000
    inp = W.make_inputs(sh, T, seed=11, device=DEV, routing="replay", weights=w235)
    gate, up = W.packed_views(inp["w13"], sh.inter)
    ids, w = inp["topk_ids"], inp["topk_weights"]
    q = moe.moe_query_config(inp["x"], gate, up, inp["w2"], ids, w)
    out = moe.moe_fused_fwd(inp["x"], gate, up, inp["w2"], ids, w).clone()
    for t0, n in ((32768, 32768), (65536, T - 65536)):
        part = moe.moe_fused_fwd(inp["x"][t0:t0 + n], gate, up, inp["w2"], ids[t0:t0 + n], w[t0:t0 + n],
                                 force_config=q["config_index"])
        assert torch.equal(part, out[t0:t0 + n]), t0
    _check_bf16(inp, out, np_(ids), np_(w), tail_tokens(np_(ids), sh.experts, 256))


def test_mxfp4_beyond_largest_bucket(fp4_weights):
    """70000 tokens on the 512/10 MXFP4 shard, past the largest bucket (the
    32768 bucket's configuration, 5.7 GB of per-slot rows written through
    64-bit offsets, the multi-launch align at 700000 assignments): slices of
    the tokens run alone give the same rows bit for bit, and sampled tokens,
    including the experts' ragged tail blocks, match the oracle."""
    shape = W.QWEN35_397B_TP2_FP4_512
    w13, w2, ((gq, gs), (uq, us), (wq, wsc)) = fp4_weights(shape)
    T = 70000
    inp = W.make_inputs(shape, T, seed=13, device=DEV, weights=(w13, w2))
    gpu, orc = route_both(inp)
    assert_routing_equal(gpu, orc)
    kw = dict(gate_scale=gs, up_scale=us, w2_scale=wsc, mode=moe.MODE_MXFP4)
    q = moe.moe_query_config(inp["x"], gq, uq, wq, *gpu, **kw)
    out = moe.moe_fused_fwd(inp["x"], gq, uq, wq, *gpu, **kw).clone()
    ids, w = gpu
    for t0, n in ((32768, 32768), (65536, T - 65536)):
        part = moe.moe_fused_fwd(inp["x"][t0:t0 + n], gq, uq, wq, ids[t0:t0 + n], w[t0:t0 + n],
                                 force_config=q["config_index"], **kw)
        assert torch.equal(part, out[t0:t0 + n]), t0
    oi, ow = orc
    toks = tail_tokens(oi, shape.experts, 128)
    mx = fp4_weights.oracle_codes(shape, sorted({int(e) for e in oi[toks].ravel()}))
    acc, _ = oracle_ffn_tokens(inp, oi, ow, toks, mx=mx)
    got = bf16_to_f64(out[torch.from_numpy(toks).to(DEV)])
    r, er = rel_l2(got, acc), err_ratio(got, acc)
    print(f"T={T} {len(toks)} tokens rel_l2={r:.3e} err_ratio={er:.3e}")
    assert np.isfinite(got).all()
    assert r <= FP4_TOL and er <= FP4_ERR_RATIO
