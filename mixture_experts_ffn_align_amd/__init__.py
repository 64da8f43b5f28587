"""Fused MoE expert-FFN forward for MI355X (gfx950) — Python binding.

Thin marshalling over the C ABI in ``include/moeffn.h`` (``libmoeffn.so``):
torch tensors become strided descriptors, the current torch stream becomes the
launch stream, and every step runs in the library's HIP kernels. torch is used
for device memory and streams only. The function names match the C entry
points.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import _abi
from ._abi import (DT_BF16, DT_E8M0, DT_F32, DT_FP4X2, DT_I32, MODE_BF16, MODE_MXFP4, STAGES,
                   MoEError)

__all__ = ["moe_topk_softmax", "moe_align", "moe_align_capacity", "moe_quant_mxfp4",
           "moe_fused_fwd", "moe_fused_fwd_noalloc", "moe_fused_workspace_size", "moe_query_config",
           "moe_combine",
           "moe_rmsnorm", "moe_fused_bwd", "moe_fused_bwd_workspace_size", "MoEError",
           "MODE_BF16", "MODE_MXFP4", "STAGES", "library_path"]

_TORCH_DT = {torch.bfloat16: DT_BF16, torch.float32: DT_F32, torch.int32: DT_I32}


def library_path() -> str:
    return _abi.LIB_PATH


def _desc(t: Optional[torch.Tensor], dtype: Optional[int] = None) -> _abi.TensorDesc:
    d = _abi.TensorDesc()
    if t is None:
        return d
    if dtype is None:
        if t.dtype not in _TORCH_DT:
            raise TypeError(f"no descriptor type for {t.dtype}")
        dtype = _TORCH_DT[t.dtype]
    elif dtype in (DT_FP4X2, DT_E8M0) and t.dtype != torch.uint8:
        raise TypeError("fp4x2 / e8m0 tensors travel as torch.uint8")
    if t.dim() > _abi.MOE_MAX_DIMS:
        raise ValueError("too many dims")
    d.data = t.data_ptr() if t.numel() > 0 else 0
    d.dtype = dtype
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.size[i] = t.size(i)
        d.stride[i] = t.stride(i)
    return d


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def moe_topk_softmax(logits: torch.Tensor, k: int, renorm: bool = True, shared_id: int = -1,
                     shared_w: float = 1.0, ids: Optional[torch.Tensor] = None,
                     weights: Optional[torch.Tensor] = None, stream=None):
    """Router: ids [T, k(+1)] int32 and weights [T, k(+1)] fp32 (any strides)."""
    L = _abi.load()
    T = logits.shape[0]
    kt = k + (1 if shared_id >= 0 else 0)
    if ids is None:
        ids = torch.empty((T, kt), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((T, kt), dtype=torch.float32, device=logits.device)
    dl, di, dw = _desc(logits), _desc(ids), _desc(weights)
    _abi.check(L.moe_topk_softmax(ctypes.byref(dl), k, int(renorm), shared_id, float(shared_w),
                                  ctypes.byref(di), ctypes.byref(dw), _stream(stream)))
    return ids, weights


def moe_align_capacity(assignments: int, num_experts: int, block_m: int) -> int:
    return int(_abi.load().moe_align_capacity(assignments, num_experts, block_m))


def moe_align(ids: torch.Tensor, num_experts: int, block_m: int, stream=None):
    """Stable align by expert: (sorted_ids [cap], block_expert [cap/bm], n_padded [1])."""
    L = _abi.load()
    T, k = ids.shape
    cap = moe_align_capacity(T * k, num_experts, block_m)
    dev = ids.device
    sorted_ids = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    block_expert = torch.empty(max(cap // block_m, 1), dtype=torch.int32, device=dev)
    n_padded = torch.empty(1, dtype=torch.int32, device=dev)
    nbytes = ctypes.c_size_t(0)
    _abi.check(L.moe_align_workspace_size(T, k, num_experts, block_m, ctypes.byref(nbytes)))
    ws = torch.empty(max(nbytes.value, 256), dtype=torch.uint8, device=dev)
    di, ds, db, dn = _desc(ids), _desc(sorted_ids), _desc(block_expert), _desc(n_padded)
    _abi.check(L.moe_align(ctypes.byref(di), num_experts, block_m, ctypes.byref(ds), ctypes.byref(db),
                           ctypes.byref(dn), ws.data_ptr(), ws.numel(), _stream(stream)))
    return sorted_ids, block_expert, n_padded


def moe_quant_mxfp4(src: torch.Tensor, codes: Optional[torch.Tensor] = None,
                    scales: Optional[torch.Tensor] = None, stream=None):
    """bf16 [.., K] (any strides) -> (codes uint8 [.., K/2], scales uint8 [.., K/32])."""
    L = _abi.load()
    K = src.shape[-1]
    lead = tuple(src.shape[:-1])
    if codes is None:
        codes = torch.empty(lead + (K // 2,), dtype=torch.uint8, device=src.device)
    if scales is None:
        scales = torch.empty(lead + (K // 32,), dtype=torch.uint8, device=src.device)
    d0, d1, d2 = _desc(src), _desc(codes, DT_FP4X2), _desc(scales, DT_E8M0)
    _abi.check(L.moe_quant_mxfp4(ctypes.byref(d0), ctypes.byref(d1), ctypes.byref(d2), _stream(stream)))
    return codes, scales


def _fused_args(x, gate, up, w2, topk_ids, topk_weights, out, gate_scale=None, up_scale=None,
                w2_scale=None, mode=MODE_BF16, stage_events=None, force_config=-1, expert_offset=0,
                num_global_experts=0, y_rows=None, norm_weight=None, norm_eps=1e-6):
    a = _abi.FusedArgs()
    a.mode = mode
    a.activation = _abi.ACT_SILU
    wdt = DT_FP4X2 if mode == MODE_MXFP4 else DT_BF16
    a.x = _desc(x)
    a.gate, a.up, a.w2 = _desc(gate, wdt), _desc(up, wdt), _desc(w2, wdt)
    if mode == MODE_MXFP4:
        a.gate_scale = _desc(gate_scale, DT_E8M0)
        a.up_scale = _desc(up_scale, DT_E8M0)
        a.w2_scale = _desc(w2_scale, DT_E8M0)
    a.topk_ids = _desc(topk_ids)
    a.topk_weights = _desc(topk_weights)
    a.out = _desc(out)
    a.force_config = force_config
    a.expert_offset = expert_offset
    a.num_global_experts = num_global_experts
    a.y_rows = _desc(y_rows)
    a.norm_weight = _desc(norm_weight)
    a.norm_eps = float(norm_eps)
    keep = None
    if stage_events is not None:
        keep = (ctypes.c_void_p * len(stage_events))(*[e or None for e in stage_events])
        a.stage_events = ctypes.cast(keep, ctypes.c_void_p)
    return a, keep


def moe_fused_workspace_size(x, gate, up, w2, topk_ids, topk_weights, out=None, **kw) -> int:
    if out is None:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)   # shape only
    a, _ = _fused_args(x, gate, up, w2, topk_ids, topk_weights, out, **kw)
    n = ctypes.c_size_t(0)
    _abi.check(_abi.load().moe_fused_workspace_size(ctypes.byref(a), ctypes.byref(n)))
    return n.value


def moe_query_config(x, gate, up, w2, topk_ids, topk_weights, out=None, **kw) -> dict:
    if out is None:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)   # shape only
    a, _ = _fused_args(x, gate, up, w2, topk_ids, topk_weights, out, **kw)
    c = _abi.Config()
    _abi.check(_abi.load().moe_query_config(ctypes.byref(a), ctypes.byref(c)))
    return {f: getattr(c, f) for f, _ in _abi.Config._fields_}


_ws_cache: dict = {}


def _ws_get(cache: dict, key, nbytes: int, alloc):
    """The cached buffer for ``key`` if it holds ``nbytes``, else a new one
    from ``alloc`` that replaces it."""
    ws = cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = alloc(max(nbytes, 256))
        cache[key] = ws
    return ws


def _workspace(nbytes: int, device, stream: int) -> torch.Tensor:
    """The binding's default workspace for calls that pass none: one buffer
    per (device, stream), since calls that share a workspace must be ordered
    on one stream. A new buffer is marked as used on its stream
    (record_stream), so when a larger one replaces it the caching allocator
    waits for that stream's queued kernels before handing the memory out
    again. During graph capture the caller must pass a workspace of its own:
    a replayed graph would keep writing into a buffer this cache may drop."""
    if torch.cuda.is_current_stream_capturing():
        raise MoEError(-5, "pass workspace= explicitly when capturing a graph")
    dev = torch.device(device)
    if dev.index is None:
        dev = torch.device(dev.type, torch.cuda.current_device())
    st = int(stream)

    def alloc(n):
        ws = torch.empty(n, dtype=torch.uint8, device=dev)
        use = torch.cuda.default_stream(dev) if st == 0 else torch.cuda.ExternalStream(st, device=dev)
        if use.cuda_stream != torch.cuda.current_stream(dev).cuda_stream:
            ws.record_stream(use)
        return ws
    return _ws_get(_ws_cache, (dev.type, dev.index, st), nbytes, alloc)


def moe_fused_fwd(x: torch.Tensor, gate: torch.Tensor, up: torch.Tensor, w2: torch.Tensor,
                  topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                  out: Optional[torch.Tensor] = None, *, gate_scale=None, up_scale=None,
                  w2_scale=None, mode: int = MODE_BF16, workspace: Optional[torch.Tensor] = None,
                  stage_events: Optional[Sequence[int]] = None, force_config: int = -1,
                  expert_offset: int = 0, num_global_experts: int = 0,
                  y_rows: Optional[torch.Tensor] = None, norm_weight: Optional[torch.Tensor] = None,
                  norm_eps: float = 1e-6, stream=None) -> torch.Tensor:
    """Fused MoE forward: align, (quantise x), gemm1 + SiLU*up, gemm2, combine.

    bf16 mode: gate/up [E, I, H] and w2 [E, H, I] bf16 (any expert/row strides).
    MXFP4 mode: gate/up/w2 are uint8 code tensors [.., K/2] with uint8 e8m0
    scales [.., K/32]. stage_events: 10 raw hipEvent_t handles (0 skips one) or None.
    Expert-parallel shard: the weights hold global experts expert_offset ..
    expert_offset + E - 1 of num_global_experts; other slots are skipped. With
    y_rows ([T, k, H] bf16) the per-slot results of local slots go there and
    the call returns y_rows without combining. norm_weight ([H] bf16 or fp32):
    gemm1 reads moe_rmsnorm(x, norm_weight, norm_eps) instead of x.
    """
    L = _abi.load()
    if out is None and y_rows is None:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    a, keep = _fused_args(x, gate, up, w2, topk_ids, topk_weights, out, gate_scale, up_scale,
                          w2_scale, mode, stage_events, force_config, expert_offset,
                          num_global_experts, y_rows, norm_weight, norm_eps)
    n = ctypes.c_size_t(0)
    _abi.check(L.moe_fused_workspace_size(ctypes.byref(a), ctypes.byref(n)))
    st = _stream(stream)
    if workspace is None:
        workspace = _workspace(n.value, x.device, st)
    _abi.check(L.moe_fused_fwd(ctypes.byref(a), workspace.data_ptr() if workspace.numel() else 0,
                               workspace.numel(), st))
    del keep
    return y_rows if y_rows is not None else out


def moe_fused_fwd_noalloc(x: torch.Tensor, gate: torch.Tensor, up: torch.Tensor, w2: torch.Tensor,
                          topk_ids: torch.Tensor, topk_weights: torch.Tensor, out: torch.Tensor, *,
                          gate_scale=None, up_scale=None, w2_scale=None, mode: int = MODE_BF16,
                          force_config: int = -1, expert_offset: int = 0, num_global_experts: int = 0,
                          y_rows: Optional[torch.Tensor] = None, norm_weight: Optional[torch.Tensor] = None,
                          norm_eps: float = 1e-6, stream=None) -> torch.Tensor:
    """moe_fused_fwd on the library's built-in device scratch: no workspace and
    no allocation, for callers that cannot allocate (out, or y_rows, must be
    given). Calls that overlap on one GPU race on that scratch."""
    L = _abi.load()
    if out is None and y_rows is None:
        raise ValueError("moe_fused_fwd_noalloc needs out (or y_rows): it allocates nothing")
    a, keep = _fused_args(x, gate, up, w2, topk_ids, topk_weights, out, gate_scale, up_scale, w2_scale, mode,
                          None, force_config, expert_offset, num_global_experts, y_rows, norm_weight, norm_eps)
    _abi.check(L.moe_fused_fwd_noalloc(ctypes.byref(a), _stream(stream)))
    del keep
    return y_rows if y_rows is not None else out


def _bwd_args(x, gate, up, w2, topk_ids, topk_weights, dout, dx, dgate, dup, dw2, dtopk_weights,
              expert_offset=0, num_global_experts=0, accumulate=False):
    b = _abi.BwdArgs()
    fa, _ = _fused_args(x, gate, up, w2, topk_ids, topk_weights, dx, expert_offset=expert_offset,
                        num_global_experts=num_global_experts)
    b.fwd = fa
    b.dout, b.dx = _desc(dout), _desc(dx)
    b.dgate, b.dup, b.dw2 = _desc(dgate), _desc(dup), _desc(dw2)
    b.dtopk_weights = _desc(dtopk_weights)
    b.accumulate = int(bool(accumulate))
    return b


def moe_fused_bwd_workspace_size(x, gate, up, w2, topk_ids, topk_weights, dout, *, grad_dtype=torch.float32,
                                 expert_offset=0, num_global_experts=0) -> int:
    E, I, H = gate.shape
    T, k = topk_ids.shape
    dev = x.device
    shapes = [torch.empty(x.shape, dtype=torch.bfloat16, device=dev),
              torch.empty((E, I, H), dtype=grad_dtype, device=dev), torch.empty((E, I, H), dtype=grad_dtype, device=dev),
              torch.empty((E, H, I), dtype=grad_dtype, device=dev), torch.empty((T, k), dtype=torch.float32, device=dev)]
    b = _bwd_args(x, gate, up, w2, topk_ids, topk_weights, dout, *shapes, expert_offset=expert_offset,
                  num_global_experts=num_global_experts)
    n = ctypes.c_size_t(0)
    _abi.check(_abi.load().moe_fused_bwd_workspace_size(ctypes.byref(b), ctypes.byref(n)))
    return n.value


def moe_fused_bwd(x, gate, up, w2, topk_ids, topk_weights, dout, *, dx=None, dgate=None, dup=None, dw2=None,
                  dtopk_weights=None, grad_dtype=torch.float32, expert_offset: int = 0,
                  num_global_experts: int = 0, accumulate: bool = False,
                  workspace: Optional[torch.Tensor] = None, stream=None):
    """Gradients of sum(dout * out) for the bf16 fused forward.

    Returns (dx [T, H] bf16, dgate [E, I, H], dup [E, I, H], dw2 [E, H, I] in
    grad_dtype (float32 or bfloat16), dtopk_weights [T, k] float32). Outputs
    may be passed in with any allowed strides (dgate/dup as views of one
    packed dw13 [E, 2I, H], for instance). accumulate=True adds the weight
    gradients into the given dgate/dup/dw2 and leaves experts without slots
    untouched.
    """
    L = _abi.load()
    E, I, H = gate.shape
    T, k = topk_ids.shape
    dev = x.device
    if dx is None:
        dx = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if dgate is None:
        dgate = torch.empty((E, I, H), dtype=grad_dtype, device=dev)
    if dup is None:
        dup = torch.empty((E, I, H), dtype=grad_dtype, device=dev)
    if dw2 is None:
        dw2 = torch.empty((E, H, I), dtype=grad_dtype, device=dev)
    if dtopk_weights is None:
        dtopk_weights = torch.empty((T, k), dtype=torch.float32, device=dev)
    b = _bwd_args(x, gate, up, w2, topk_ids, topk_weights, dout, dx, dgate, dup, dw2, dtopk_weights,
                  expert_offset, num_global_experts, accumulate)
    n = ctypes.c_size_t(0)
    _abi.check(L.moe_fused_bwd_workspace_size(ctypes.byref(b), ctypes.byref(n)))
    st = _stream(stream)
    if workspace is None:
        workspace = _workspace(n.value, dev, st)
    _abi.check(L.moe_fused_bwd(ctypes.byref(b), workspace.data_ptr() if workspace.numel() else 0,
                               workspace.numel(), st))
    return dx, dgate, dup, dw2, dtopk_weights


def moe_rmsnorm(x: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6,
                out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out[t] = bf16((x[t] * r_t) * weight), r_t = 1/sqrt(mean(x[t]^2) + eps), fp32 inside."""
    L = _abi.load()
    if out is None:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    dx, dw, do = _desc(x), _desc(weight), _desc(out)
    _abi.check(L.moe_rmsnorm(ctypes.byref(dx), ctypes.byref(dw), float(eps), ctypes.byref(do), _stream(stream)))
    return out


def moe_combine(y_rows: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                num_experts: int, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out[t] = bf16(slot-ordered fmaf sum of w[t, j] * y_rows[t, j]) over ids in [0, num_experts)."""
    L = _abi.load()
    T, _, H = y_rows.shape
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y_rows.device)
    dy, di, dw, do = _desc(y_rows), _desc(topk_ids), _desc(topk_weights), _desc(out)
    _abi.check(L.moe_combine(ctypes.byref(dy), ctypes.byref(di), ctypes.byref(dw), num_experts,
                             ctypes.byref(do), _stream(stream)))
    return out
