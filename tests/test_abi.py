"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and its host-side checks reject bad arguments before any launch
(no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest
import torch

import mixture_experts_ffn_align_amd as moe
from mixture_experts_ffn_align_amd import _abi
from mixture_experts_ffn_align_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moeffn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    L = _abi.load()
    names = _declared()
    assert set(names) == set(_abi.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_strerror_covers_all_codes():
    L = _abi.load()
    for code in _abi.STATUS:
        assert L.moe_strerror(code)
    assert L.moe_strerror(12345) == b"unknown status"


def _bf16_case(T=8, H=256, I=128, E=8, k=2):
    x = torch.zeros(T, H, dtype=torch.bfloat16)
    w13 = torch.zeros(E, 2 * I, H, dtype=torch.bfloat16)
    w2 = torch.zeros(E, H, I, dtype=torch.bfloat16)
    ids = torch.zeros(T, k, dtype=torch.int32)
    w = torch.zeros(T, k, dtype=torch.float32)
    gate, up = W.packed_views(w13, I)
    return x, gate, up, w2, ids, w


def _status(fn):
    with pytest.raises(moe.MoEError) as ei:
        fn()
    return _abi.STATUS[ei.value.status]


def test_shape_errors_name_the_argument():
    x, gate, up, w2, ids, w = _bf16_case()
    bad_gate = torch.zeros(8, 128, 128, dtype=torch.bfloat16)          # hidden 128 != 256
    st = _status(lambda: moe.moe_fused_workspace_size(x, bad_gate, up, w2, ids, w))
    assert st == "MOE_ERR_SHAPE"
    assert "gate" in _abi.load().moe_last_error().decode()
    assert _status(lambda: moe.moe_fused_workspace_size(x, gate, up[:4], w2, ids, w)) == "MOE_ERR_SHAPE"
    assert _status(lambda: moe.moe_fused_workspace_size(x, gate, up, w2, ids[:, :1], w)) == "MOE_ERR_SHAPE"


def test_dtype_and_layout_errors():
    x, gate, up, w2, ids, w = _bf16_case()
    assert _status(lambda: moe.moe_fused_workspace_size(x.float(), gate, up, w2, ids, w)) == "MOE_ERR_DTYPE"
    assert _status(lambda: moe.moe_fused_workspace_size(x, gate, up, w2, ids.float(), w)) == "MOE_ERR_DTYPE"
    # weight last-dim stride must be 1
    gt = torch.zeros(8, 256, 128, dtype=torch.bfloat16).transpose(1, 2)   # [8, 128, 256], stride (.., 1, 128)
    assert _status(lambda: moe.moe_fused_workspace_size(x, gt, up, w2, ids, w)) == "MOE_ERR_LAYOUT"
    # rows not on 16-byte boundaries
    buf = torch.zeros(8, 128, 260, dtype=torch.bfloat16)
    assert _status(lambda: moe.moe_fused_workspace_size(x, buf[:, :, :256], up, w2, ids, w)) == "MOE_ERR_LAYOUT"
    # output overlapping an input
    st = _status(lambda: moe.moe_query_config(x, gate, up, w2, ids, w, out=x))
    assert st == "MOE_ERR_LAYOUT"


def test_unsupported_sizes():
    x, gate, up, w2, ids, w = _bf16_case(E=2000)
    assert _status(lambda: moe.moe_fused_workspace_size(x, gate, up, w2, ids, w)) == "MOE_ERR_UNSUPPORTED"
    x, gate, up, w2, ids, w = _bf16_case(I=48)
    assert _status(lambda: moe.moe_fused_workspace_size(x, gate, up, w2, ids, w)) == "MOE_ERR_UNSUPPORTED"


def test_workspace_too_small_is_rejected_before_launch():
    x, gate, up, w2, ids, w = _bf16_case()
    ws = torch.zeros(256, dtype=torch.uint8)
    st = _status(lambda: moe.moe_fused_fwd(x, gate, up, w2, ids, w, workspace=ws, stream=0))
    assert st == "MOE_ERR_WORKSPACE"


def test_empty_batch_returns_ok_without_launch():
    x, gate, up, w2, ids, w = _bf16_case(T=0)
    out = moe.moe_fused_fwd(x, gate, up, w2, ids, w, workspace=torch.zeros(256, dtype=torch.uint8),
                            stream=0)
    assert out.shape == (0, 256)


def test_mxfp4_shapes_and_k_multiple():
    T, H, I, E = 4, 256, 256, 4
    x = torch.zeros(T, H, dtype=torch.bfloat16)
    gq = torch.zeros(E, I, H // 2, dtype=torch.uint8)
    gs = torch.zeros(E, I, H // 32, dtype=torch.uint8)
    wq = torch.zeros(E, H, I // 2, dtype=torch.uint8)
    ws_ = torch.zeros(E, H, I // 32, dtype=torch.uint8)
    ids = torch.zeros(T, 2, dtype=torch.int32)
    w = torch.zeros(T, 2, dtype=torch.float32)
    n = moe.moe_fused_workspace_size(x, gq, gq.clone(), wq, ids, w, gate_scale=gs, up_scale=gs.clone(),
                                     w2_scale=ws_, mode=moe.MODE_MXFP4)
    assert n > 0
    st = _status(lambda: moe.moe_fused_workspace_size(x, gq, gq.clone(), wq, ids, w, gate_scale=gs[:, :, :4],
                                                      up_scale=gs.clone(), w2_scale=ws_, mode=moe.MODE_MXFP4))
    assert st == "MOE_ERR_SHAPE"
    x2 = torch.zeros(T, 192, dtype=torch.bfloat16)                 # 192 is not a multiple of 256
    g2 = torch.zeros(E, I, 96, dtype=torch.uint8)
    s2 = torch.zeros(E, I, 6, dtype=torch.uint8)
    w22 = torch.zeros(E, 192, I // 2, dtype=torch.uint8)
    s22 = torch.zeros(E, 192, I // 32, dtype=torch.uint8)
    st = _status(lambda: moe.moe_fused_workspace_size(x2, g2, g2.clone(), w22, ids, w, gate_scale=s2,
                                                      up_scale=s2.clone(), w2_scale=s22, mode=moe.MODE_MXFP4))
    assert st == "MOE_ERR_UNSUPPORTED"


def test_workspace_does_not_depend_on_weight_strides():
    """No weight copy is ever made: packed views and contiguous copies need the
    same workspace and get the same configuration (the copies the Liger PR
    measured at 0.375 GiB per layer do not exist here)."""
    x, gate, up, w2, ids, w = _bf16_case(T=64)
    a = moe.moe_fused_workspace_size(x, gate, up, w2, ids, w)
    b = moe.moe_fused_workspace_size(x, gate.contiguous(), up.contiguous(), w2, ids, w)
    assert a == b
    assert moe.moe_query_config(x, gate, up, w2, ids, w) == moe.moe_query_config(
        x, gate.contiguous(), up.contiguous(), w2, ids, w)
    # x stored transposed needs one re-layout buffer of T*H bf16 and nothing else
    xt = x.t().contiguous().t()
    c = moe.moe_fused_workspace_size(xt, gate, up, w2, ids, w)
    assert a < c <= a + 64 * 256 * 2 + 256


def test_config_depends_on_bucket_only():
    cfgs = []
    for T in (1, 2, 16, 17, 32, 512):
        x, gate, up, w2, ids, w = _bf16_case(T=T)
        cfgs.append(moe.moe_query_config(x, gate, up, w2, ids, w))
    assert cfgs[0]["bucket"] == 1 and cfgs[3]["bucket"] == 32 and cfgs[-1]["bucket"] == 512
    assert cfgs[3] == cfgs[4]


def test_align_and_route_argument_checks():
    ids = torch.zeros(4, 2, dtype=torch.int32)
    L = _abi.load()
    assert L.moe_align_capacity(8, 8, 16) == 128
    assert L.moe_align_capacity(0, 8, 16) == 0
    assert L.moe_align_capacity(8, 8, 24) == -1
    st = _status(lambda: moe.moe_align(ids, 8, 24))
    assert st == "MOE_ERR_ARG"
    logits = torch.zeros(4, 8)
    st = _status(lambda: moe.moe_topk_softmax(logits, 9, stream=0))
    assert st == "MOE_ERR_ARG"
    st = _status(lambda: moe.moe_topk_softmax(logits, 2, ids=torch.zeros(4, 3, dtype=torch.int32),
                                              stream=0))
    assert st == "MOE_ERR_SHAPE"
    nb = ctypes.c_size_t(0)
    assert L.moe_align_workspace_size(4, 2, 8, 16, ctypes.byref(nb)) == 0 and nb.value == 0
    assert L.moe_align_workspace_size(40000, 8, 128, 16, ctypes.byref(nb)) == 0 and nb.value > 0


def test_expert_parallel_shard_checks():
    """Expert-parallel shard arguments are checked on the host: a negative
    offset or a global expert count below offset + E is MOE_ERR_ARG, a y_rows
    tensor the gemm2 epilogue cannot write is MOE_ERR_LAYOUT, and with y_rows
    the call needs no y segment of its own in the workspace."""
    T, H, k = 8, 256, 2
    x, gate, up, w2, ids, w = _bf16_case(T=T, H=H, k=k)
    st = _status(lambda: moe.moe_fused_workspace_size(x, gate, up, w2, ids, w, expert_offset=-1))
    assert st == "MOE_ERR_ARG"
    st = _status(lambda: moe.moe_fused_workspace_size(x, gate, up, w2, ids, w, expert_offset=8,
                                                      num_global_experts=15))
    assert st == "MOE_ERR_ARG"
    plain = moe.moe_fused_workspace_size(x, gate, up, w2, ids, w)
    y = torch.zeros(T, k, H, dtype=torch.bfloat16)
    with_y = moe.moe_fused_workspace_size(x, gate, up, w2, ids, w, expert_offset=8,
                                          num_global_experts=16, y_rows=y)
    assert with_y <= plain - T * k * H * 2
    # padded rows are fine, slot-major rows or a transposed last dim are not
    ypad = torch.zeros(T, k, H + 64, dtype=torch.bfloat16)[:, :, :H]
    moe.moe_fused_workspace_size(x, gate, up, w2, ids, w, y_rows=ypad)
    yslot = torch.zeros(k, T, H, dtype=torch.bfloat16).transpose(0, 1)
    assert _status(lambda: moe.moe_fused_workspace_size(x, gate, up, w2, ids, w, y_rows=yslot)) == \
        "MOE_ERR_LAYOUT"
    yt = torch.zeros(T, H, k, dtype=torch.bfloat16).transpose(1, 2)
    assert _status(lambda: moe.moe_fused_workspace_size(x, gate, up, w2, ids, w, y_rows=yt)) == \
        "MOE_ERR_LAYOUT"
    # the global expert count, not the shard's, picks the tiles
    xb, gb, ub, w2b, idb, wb = _bf16_case(T=512, H=H, E=8, k=8)
    shard = moe.moe_query_config(xb, gb, ub, w2b, idb, wb, expert_offset=0, num_global_experts=128)
    xg, gg, ug, w2g, idg, wg = _bf16_case(T=512, H=H, E=128, k=8)
    assert shard == moe.moe_query_config(xg, gg, ug, w2g, idg, wg)


def test_combine_argument_checks():
    T, k, H = 4, 2, 256
    y = torch.zeros(T, k, H, dtype=torch.bfloat16)
    ids = torch.zeros(T, k, dtype=torch.int32)
    w = torch.zeros(T, k, dtype=torch.float32)
    assert _status(lambda: moe.moe_combine(y, ids[:, :1], w, 8, stream=0)) == "MOE_ERR_SHAPE"
    assert _status(lambda: moe.moe_combine(y, ids, w, 0, stream=0)) == "MOE_ERR_ARG"
    assert _status(lambda: moe.moe_combine(y[:, :, 1:253], ids, w, 8, stream=0)) == "MOE_ERR_LAYOUT"
    assert _status(lambda: moe.moe_combine(y.float(), ids, w, 8, stream=0)) == "MOE_ERR_DTYPE"
    out = moe.moe_combine(y[:0], ids[:0], w[:0], 8, stream=0)
    assert out.shape == (0, H)


def test_rmsnorm_argument_checks():
    x, gate, up, w2, ids, w = _bf16_case(T=8, H=256)
    nw = torch.ones(256, dtype=torch.bfloat16)
    base = moe.moe_fused_workspace_size(x, gate, up, w2, ids, w)
    with_norm = moe.moe_fused_workspace_size(x, gate, up, w2, ids, w, norm_weight=nw)
    assert with_norm == base + 8 * 256 * 2          # one bf16 [T, H] segment (a multiple of 256 bytes)
    assert _status(lambda: moe.moe_fused_workspace_size(x, gate, up, w2, ids, w, norm_weight=nw[:128])) == \
        "MOE_ERR_SHAPE"
    assert _status(lambda: moe.moe_fused_workspace_size(x, gate, up, w2, ids, w,
                                                        norm_weight=nw.to(torch.int32))) == "MOE_ERR_DTYPE"
    assert _status(lambda: moe.moe_fused_workspace_size(x, gate, up, w2, ids, w, norm_weight=nw,
                                                        norm_eps=-1.0)) == "MOE_ERR_ARG"
    moe.moe_fused_workspace_size(x, gate, up, w2, ids, w, norm_weight=nw.float())
    assert _status(lambda: moe.moe_rmsnorm(torch.zeros(4, 12, dtype=torch.bfloat16),
                                           torch.ones(12), 1e-6, stream=0)) == "MOE_ERR_UNSUPPORTED"
    assert _status(lambda: moe.moe_rmsnorm(torch.zeros(4, 16, dtype=torch.bfloat16),
                                           torch.ones(8), 1e-6, stream=0)) == "MOE_ERR_SHAPE"
    xs = torch.zeros(4, 16, dtype=torch.bfloat16)
    assert _status(lambda: moe.moe_rmsnorm(xs, torch.ones(16), 1e-6, out=xs, stream=0)) == "MOE_ERR_LAYOUT"
    assert moe.moe_rmsnorm(torch.zeros(0, 16, dtype=torch.bfloat16), torch.ones(16), stream=0).shape == (0, 16)


def test_backward_argument_checks():
    x, gate, up, w2, ids, w = _bf16_case(T=8, H=256, I=128)
    dout = torch.zeros(8, 256, dtype=torch.bfloat16)
    n = moe.moe_fused_bwd_workspace_size(x, gate, up, w2, ids, w, dout)
    assert n >= 8 * 2 * (2 * 128 * 4 + 128 * 4 + 2 * 128 * 2 + 128 * 2 + 256 * 4)
    E, I, H = 8, 128, 256
    f32 = dict(dgate=torch.zeros(E, I, H), dup=torch.zeros(E, I, H), dw2=torch.zeros(E, H, I))
    assert _status(lambda: moe.moe_fused_bwd(x, gate, up, w2, ids, w, dout, stream=0,
                                             **dict(f32, dw2=torch.zeros(E, H, I, dtype=torch.bfloat16)))) == \
        "MOE_ERR_DTYPE"
    assert _status(lambda: moe.moe_fused_bwd(x, gate, up, w2, ids, w, dout, stream=0,
                                             **dict(f32, dgate=torch.zeros(E, I, H)[:, :, :H - 8]))) == \
        "MOE_ERR_SHAPE"
    assert _status(lambda: moe.moe_fused_bwd(x, gate, up, w2, ids, w, dout, dx=dout, stream=0, **f32)) == \
        "MOE_ERR_LAYOUT"
    dw13 = torch.zeros(E, 2 * I, H)
    assert _status(lambda: moe.moe_fused_bwd(x, gate, up, w2, ids, w, dout, stream=0, dgate=dw13[:, :I + 8],
                                             dup=dw13[:, I:], dw2=f32["dw2"])) == "MOE_ERR_SHAPE"
    # the halves of one packed dw13 are accepted, overlapping outputs are not
    n2 = moe.moe_fused_bwd_workspace_size(x, gate, up, w2, ids, w, dout)
    assert n2 == n
    assert _status(lambda: moe.moe_fused_bwd(x, gate, up, w2, ids, w, dout, stream=0, dgate=dw13[:, :I + 1][:, 1:],
                                             dup=dw13[:, :I], dw2=f32["dw2"])) == "MOE_ERR_LAYOUT"
    xs, gs, us, w2s, ids_s, w_s = _bf16_case(T=8, H=192, I=128)
    assert _status(lambda: moe.moe_fused_bwd_workspace_size(xs, gs, us, w2s, ids_s, w_s,
                                                            torch.zeros(8, 192, dtype=torch.bfloat16))) == \
        "MOE_ERR_UNSUPPORTED"                                   # H = 192 is not a multiple of 128


def test_backward_packed_dw13_halves_accepted():
    """dgate/dup as w13-style halves of one [E, 2I, H] gradient interleave in
    memory without sharing an element: accepted. Halves shifted so that their
    rows meet: rejected."""
    E, I, H, T, k = 8, 128, 256, 8, 2
    x, gate, up, w2, ids, w = _bf16_case(T=T, H=H, I=I, E=E, k=k)
    dout = torch.zeros(T, H, dtype=torch.bfloat16)
    dx = torch.zeros(T, H, dtype=torch.bfloat16)
    dw13 = torch.zeros(E, 2 * I, H)

    def size(dg, du):
        b = moe._bwd_args(x, gate, up, w2, ids, w, dout, dx, dg, du, torch.zeros(E, H, I), torch.zeros(T, k))
        n = ctypes.c_size_t(0)
        return _abi.load().moe_fused_bwd_workspace_size(ctypes.byref(b), ctypes.byref(n))

    assert size(dw13[:, :I], dw13[:, I:]) == 0
    assert size(dw13[:, I:], dw13[:, :I]) == 0
    assert _abi.STATUS[size(dw13[:, :I], dw13[:, I - 8:2 * I - 8])] == "MOE_ERR_LAYOUT"


def test_binding_workspace_cache_is_per_device_and_stream():
    """The binding's default workspace: one buffer per (device, stream) key,
    reused while large enough, replaced when a call needs more; other keys
    untouched (calls on different streams never share a buffer)."""
    from mixture_experts_ffn_align_amd import _ws_get
    cache, made = {}, []

    def alloc(n):
        made.append(n)
        return torch.empty(n, dtype=torch.uint8)
    a = _ws_get(cache, ("cuda", 0, 111), 1000, alloc)
    b = _ws_get(cache, ("cuda", 0, 222), 1000, alloc)
    assert a.data_ptr() != b.data_ptr()
    assert _ws_get(cache, ("cuda", 0, 111), 900, alloc) is a
    c = _ws_get(cache, ("cuda", 0, 111), 5000, alloc)
    assert c is not a and c.numel() == 5000 and cache[("cuda", 0, 111)] is c
    assert cache[("cuda", 0, 222)] is b
    d = _ws_get(cache, ("cuda", 1, 111), 10, alloc)
    assert d.numel() == 256 and made == [1000, 1000, 5000, 256]


def _strided_query(T, H, I, E, k, mode, **kw):
    """moe_query_config on views of small buffers (shapes only; no launch)."""
    def view(shape, dtype, row=16):
        st = [row] * (len(shape) - 1) + [1]
        return torch.empty(1 + sum((s - 1) * t for s, t in zip(shape, st)) + 64, dtype=dtype).as_strided(shape, st)
    x = view((T, H), torch.bfloat16)
    ids, w = view((T, k), torch.int32, 1), view((T, k), torch.float32, 1)
    if mode == moe.MODE_MXFP4:
        g, w2 = view((E, I, H // 2), torch.uint8), view((E, H, I // 2), torch.uint8)
        kw.update(gate_scale=view((E, I, H // 32), torch.uint8), up_scale=view((E, I, H // 32), torch.uint8),
                  w2_scale=view((E, H, I // 32), torch.uint8))
    else:
        g, w2 = view((E, I, H), torch.bfloat16), view((E, H, I), torch.bfloat16)
    return moe.moe_query_config(x, g, g, w2, ids, w, mode=mode, **kw)


def test_rules_take_persistent_streams_where_they_fit():
    """For an MXFP4 layer outside the tuned table (I = 512), the built-in
    rules run both GEMMs on the persistent weight streams from half a row to
    64 rows per expert, with 16-, 32- or 64-row blocks by the expected rows;
    not at fewer rows, not on tiles' ground, never in bf16 (forcing one there
    fails before any launch), nor where a workgroup per compute unit would
    get more than 256 items (forced there, it fails before any launch; the
    rules then fall back to the per-item streams)."""
    fp4 = moe.MODE_MXFP4

    def q(T, E=256, k=10, **kw):
        return _strided_query(T, 4096, 512, E, k, fp4, **kw)
    for T, bm in ((64, 16), (512, 32), (1024, 64)):
        c = q(T)
        assert (c["gemm1_kernel"], c["gemm2_kernel"], c["block_m"]) == (19, 20, bm), (T, c)
    assert q(8)["gemm1_kernel"] != 19 and q(4096)["gemm1_kernel"] != 19
    pers = q(64)["config_index"]
    bf = _strided_query(64, 4096, 512, 256, 10, moe.MODE_BF16)
    assert bf["gemm1_kernel"] != 19 and bf["gemm2_kernel"] != 20
    with pytest.raises(moe.MoEError) as ei:
        _strided_query(64, 4096, 512, 256, 10, moe.MODE_BF16, force_config=pers)
    assert ei.value.status == -6
    # 32768 tokens, top-32 of 1024 experts in 16-row blocks: over a million
    # gemm2 items, far more than 256 per compute unit
    with pytest.raises(moe.MoEError) as ei:
        q(32768, E=1024, k=32, force_config=pers)
    assert ei.value.status == -6


def test_mxfp4_register_gemm2_falls_back_past_4gb_of_y():
    """An MXFP4 layer's built-in choice at many tokens keeps h rows in
    registers for gemm2 (family 18); where the y rows would span 4 GB or more
    (the kernel addresses them with 32-bit buffer offsets) the planner takes
    the LDS tile with the same block rows instead, and a forced config that
    cannot run fails before any launch."""
    def q(T, **kw):
        H, I, E, k = 4096, 512, 256, 10     # a layer outside the tuned table: the built-in rules
        def view(shape, dtype, row=16):
            n = len(shape)
            st = [row] * (n - 1) + [1]
            return torch.empty(1 + sum((s - 1) * t for s, t in zip(shape, st)) + 64, dtype=dtype).as_strided(shape, st)
        x = view((T, H), torch.bfloat16)
        g = view((E, I, H // 2), torch.uint8)
        w2 = view((E, H, I // 2), torch.uint8)
        sc = dict(gate_scale=view((E, I, H // 32), torch.uint8), up_scale=view((E, I, H // 32), torch.uint8),
                  w2_scale=view((E, H, I // 32), torch.uint8), mode=moe.MODE_MXFP4)
        ids, w = view((T, k), torch.int32, 1), view((T, k), torch.float32, 1)
        out = torch.empty(T * H + 64, dtype=torch.bfloat16).as_strided((T, H), (H, 1))
        return moe.moe_query_config(x, g, g, w2, ids, w, out=out, **sc, **kw)
    assert q(32768)["gemm2_kernel"] == 18
    big = q(60000)
    assert big["gemm2_kernel"] == 14 and big["block_m2"] == big["block_m"]
    with pytest.raises(moe.MoEError) as ei:
        q(60000, force_config=41)
    assert ei.value.status == -6


def test_oversized_calls_run_in_token_chunks():
    """A bf16 Qwen3-235B-shaped call with 90000 tokens (its tiled gemm2
    operands would pass 2^31 bytes) is planned as chunks of 32768 tokens:
    accepted, with the workspace and configuration of one full chunk; a
    forced configuration that cannot take the whole call still fails."""
    def args(T, **kw):
        H, I, E, k = 4096, 1536, 128, 8
        def view(shape, dtype, row=16):
            n = len(shape)
            st = [row] * (n - 1) + [1]
            return torch.empty(1 + sum((s - 1) * t for s, t in zip(shape, st)) + 64, dtype=dtype).as_strided(shape, st)
        x = view((T, H), torch.bfloat16)
        g = view((E, I, H), torch.bfloat16)
        w2 = view((E, H, I), torch.bfloat16)
        ids, w = view((T, k), torch.int32, 1), view((T, k), torch.float32, 1)
        out = torch.empty(T * H + 64, dtype=torch.bfloat16).as_strided((T, H), (H, 1))
        return (x, g, g, w2, ids, w), dict(out=out, **kw)
    a, kw = args(90000)
    big = moe.moe_query_config(*a, **kw)
    a1, kw1 = args(32768)
    one = moe.moe_query_config(*a1, **kw1)
    assert big == one and big["bucket"] == 32768
    assert moe.moe_fused_workspace_size(*a, **kw) == moe.moe_fused_workspace_size(*a1, **kw1)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_query_config(*a, force_config=big["config_index"], **kw)
    assert ei.value.status == -6
