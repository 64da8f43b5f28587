"""CPU oracle for the fused MoE expert-FFN forward — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package. The product path (the HIP library and its
binding) never imports it, and it imports nothing from the product.

The arithmetic lives in ``moe_oracle.c`` (plain C, double precision, built
with gcc ``-O2 -fno-fast-math -ffp-contract=off``); this module only marshals
numpy arrays into it. bf16 tensors travel as ``uint16`` bit patterns, MXFP4
tensors as ``uint8`` (two e2m1 codes per byte, element 2i in the low nibble)
plus ``uint8`` e8m0 scale bytes. Strides are whatever the arrays carry.

Each function cites what it follows in its C counterpart's comment. Parity
status: route, align, mxfp4 quantisation, the FFN/combine and the RMSNorm are
pinned by the ``-m "not gpu"`` tests in ``tests/test_oracle_*.py`` (brute
force, closed forms, invariants, a dense-MLP special case and the pages'
printed numbers).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_moe.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP, no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
               "-shared", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _FfnArgs(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int32), ("round_h", ctypes.c_int32),
        ("T", ctypes.c_int64), ("H", ctypes.c_int64), ("I", ctypes.c_int64),
        ("E", ctypes.c_int64), ("k", ctypes.c_int64),
        ("x", ctypes.c_void_p), ("xs_t", ctypes.c_int64), ("xs_h", ctypes.c_int64),
        ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("w2", ctypes.c_void_p),
        ("gs_e", ctypes.c_int64), ("gs_r", ctypes.c_int64), ("gs_c", ctypes.c_int64),
        ("us_e", ctypes.c_int64), ("us_r", ctypes.c_int64), ("us_c", ctypes.c_int64),
        ("w2s_e", ctypes.c_int64), ("w2s_r", ctypes.c_int64), ("w2s_c", ctypes.c_int64),
        ("gate_q", ctypes.c_void_p), ("up_q", ctypes.c_void_p), ("w2_q", ctypes.c_void_p),
        ("gate_sc", ctypes.c_void_p), ("up_sc", ctypes.c_void_p), ("w2_sc", ctypes.c_void_p),
        ("gqs_e", ctypes.c_int64), ("gqs_r", ctypes.c_int64),
        ("uqs_e", ctypes.c_int64), ("uqs_r", ctypes.c_int64),
        ("w2qs_e", ctypes.c_int64), ("w2qs_r", ctypes.c_int64),
        ("gss_e", ctypes.c_int64), ("gss_r", ctypes.c_int64),
        ("uss_e", ctypes.c_int64), ("uss_r", ctypes.c_int64),
        ("w2ss_e", ctypes.c_int64), ("w2ss_r", ctypes.c_int64),
        ("ids", ctypes.c_void_p), ("is_t", ctypes.c_int64), ("is_j", ctypes.c_int64),
        ("wts", ctypes.c_void_p), ("ws_t", ctypes.c_int64), ("ws_j", ctypes.c_int64),
    ]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.orc_route.argtypes = [vp, i64, i64, i64, i64, i32, i32, i32, ctypes.c_float,
                                vp, i64, i64, vp, i64, i64]
        L.orc_route.restype = i32
        L.orc_align.argtypes = [vp, i64, i32, i64, i64, i32, i32, vp, vp, i64,
                                ctypes.POINTER(i64)]
        L.orc_align.restype = i32
        L.orc_mxfp4_quant_bf16.argtypes = [vp, i64, i64, i64, i64, vp, vp]
        L.orc_mxfp4_quant_bf16.restype = i32
        L.orc_mxfp4_quant.argtypes = [vp, i64, vp, vp]
        L.orc_mxfp4_quant.restype = None
        L.orc_ffn.argtypes = [ctypes.POINTER(_FfnArgs), vp, i64, vp, vp]
        L.orc_ffn.restype = i32
        L.orc_ffn_args_size.restype = i64
        L.orc_rmsnorm.argtypes = [vp, i64, i64, i64, i64, vp, i64, ctypes.c_double, vp, vp]
        L.orc_rmsnorm.restype = i32
        L.orc_ffn_bwd.argtypes = [ctypes.POINTER(_FfnArgs), vp, i64, i64, vp, i64, vp, vp, vp, vp, i64,
                                  vp, vp, vp]
        L.orc_ffn_bwd.restype = i32
        L.orc_route_exp.argtypes = [ctypes.c_double]
        L.orc_route_exp.restype = ctypes.c_double
        L.orc_e2m1_value.argtypes = [i32]
        L.orc_e2m1_value.restype = ctypes.c_double
        L.orc_e8m0_value.argtypes = [i32]
        L.orc_e8m0_value.restype = ctypes.c_double
        assert L.orc_ffn_args_size() == ctypes.sizeof(_FfnArgs), "oracle ABI mirror mismatch"
        _lib = L
    return _lib


def _es(a: np.ndarray, dim: int) -> int:
    """Stride of ``dim`` in elements."""
    s = a.strides[dim]
    assert s % a.itemsize == 0
    return s // a.itemsize


def _ptr(a: Optional[np.ndarray]) -> Optional[int]:
    return None if a is None else a.ctypes.data


# ------------------------------------------------------------------ route

def route_exp(d: float) -> float:
    """The router's stated double-precision exp(d), d <= 0 (orc_route_exp)."""
    return float(lib().orc_route_exp(float(d)))


def route(logits: np.ndarray, k: int, renorm: bool = True, shared_id: int = -1,
          shared_w: float = 1.0) -> tuple[np.ndarray, np.ndarray]:
    """Top-k of the softmax over each row of ``logits`` (fp32 [T, E]): the k
    largest logits with ties to the lower index, weights exp(l_j - l_max)
    (the stated exp) over their slot-order sum (renorm) or over the sum over
    all experts, rounded once to fp32; plus an appended shared expert."""
    assert logits.dtype == np.float32 and logits.ndim == 2
    T, E = logits.shape
    kt = k + (1 if shared_id >= 0 else 0)
    ids = np.zeros((T, kt), dtype=np.int32)
    w = np.zeros((T, kt), dtype=np.float32)
    rc = lib().orc_route(_ptr(logits), T, E, _es(logits, 0), _es(logits, 1), k, int(renorm),
                         shared_id, shared_w, _ptr(ids), kt, 1, _ptr(w), kt, 1)
    if rc != 0:
        raise ValueError("orc_route failed")
    return ids, w


# ------------------------------------------------------------------ align

def align(ids: np.ndarray, num_experts: int, block_m: int) -> tuple[np.ndarray, np.ndarray, int]:
    """Stable group-by-expert of the flat assignments, padded per expert to
    block_m with the sentinel T*k. Returns (sorted, block_expert, n_padded)."""
    assert ids.dtype == np.int32 and ids.ndim == 2
    T, k = ids.shape
    A = T * k
    cap = A + min(num_experts, max(A, 1)) * (block_m - 1) + block_m
    sorted_ = np.empty(cap, dtype=np.int32)
    be = np.empty(cap // block_m + 1, dtype=np.int32)
    n = ctypes.c_int64(0)
    rc = lib().orc_align(_ptr(ids), T, k, _es(ids, 0), _es(ids, 1), num_experts, block_m,
                         _ptr(sorted_), _ptr(be), cap, ctypes.byref(n))
    if rc != 0:
        raise ValueError("orc_align failed")
    npad = n.value
    return sorted_[:npad].copy(), be[:npad // block_m].copy(), npad


# ------------------------------------------------------------------ mxfp4

def mxfp4_quant(x_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """bf16 bits [..., K] (any strides, 2-D or 3-D) -> codes [..., K/2], scales [..., K/32]."""
    assert x_bits.dtype == np.uint16
    if x_bits.ndim == 3:
        outs = [mxfp4_quant(x_bits[e]) for e in range(x_bits.shape[0])]
        return np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs])
    R, K = x_bits.shape
    codes = np.empty((R, K // 2), dtype=np.uint8)
    scales = np.empty((R, K // 32), dtype=np.uint8)
    rc = lib().orc_mxfp4_quant_bf16(_ptr(x_bits), R, K, _es(x_bits, 0), _es(x_bits, 1),
                                    _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError("orc_mxfp4_quant_bf16 failed (K must be a multiple of 32)")
    return codes, scales


def mxfp4_quant_f32(v: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """fp32 values [n] (n a multiple of 32, contiguous) -> codes, scales."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    n = v.size
    codes = np.empty(n // 2, dtype=np.uint8)
    scales = np.empty(n // 32, dtype=np.uint8)
    lib().orc_mxfp4_quant(_ptr(v), n, _ptr(codes), _ptr(scales))
    return codes, scales


def mxfp4_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes [..., K/2], scales [..., K/32] -> float64 [..., K]."""
    L = lib()
    mags = np.array([L.orc_e2m1_value(c) for c in range(16)], dtype=np.float64)
    sc = np.array([L.orc_e8m0_value(b) for b in range(256)], dtype=np.float64)
    lo = mags[codes & 15]
    hi = mags[codes >> 4]
    vals = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    s = np.repeat(sc[scales], 32, axis=-1)
    return vals * s


# -------------------------------------------------------------------- ffn

def ffn(x_bits: np.ndarray, ids: np.ndarray, wts: np.ndarray, *, num_experts: int,
        gate: Optional[np.ndarray] = None, up: Optional[np.ndarray] = None,
        w2: Optional[np.ndarray] = None, gate_q=None, up_q=None, w2_q=None,
        toks: Optional[np.ndarray] = None, round_h: bool = True) -> tuple[np.ndarray, np.ndarray]:
    """Fused MoE forward, plain definition, for the tokens in ``toks`` (all if None).

    bf16 mode: gate/up bf16 bits [E, I, H], w2 bf16 bits [E, H, I] (any strides).
    MXFP4 mode: gate_q/up_q/w2_q = (codes, scales) pairs, codes [E, rows, K/2]
    and scales [E, rows, K/32], last dim contiguous. x is bf16 bits [T, H] (any
    strides) and is quantised to MXFP4 inside, like h.
    Returns (out_acc float64 [n, H], out_bf16 bits uint16 [n, H]).
    """
    a = _FfnArgs()
    mxfp4 = gate_q is not None
    a.mode = 1 if mxfp4 else 0
    a.round_h = int(round_h)
    T, H = x_bits.shape
    assert x_bits.dtype == np.uint16
    a.T, a.H, a.E, a.k = T, H, num_experts, ids.shape[1]
    a.x, a.xs_t, a.xs_h = _ptr(x_bits), _es(x_bits, 0), _es(x_bits, 1)
    keep = [x_bits, ids, wts]
    if not mxfp4:
        assert gate.dtype == np.uint16 and up.dtype == np.uint16 and w2.dtype == np.uint16
        a.I = gate.shape[1]
        assert gate.shape == (num_experts, a.I, H) and up.shape == gate.shape
        assert w2.shape == (num_experts, H, a.I)
        a.gate, a.up, a.w2 = _ptr(gate), _ptr(up), _ptr(w2)
        a.gs_e, a.gs_r, a.gs_c = (_es(gate, d) for d in range(3))
        a.us_e, a.us_r, a.us_c = (_es(up, d) for d in range(3))
        a.w2s_e, a.w2s_r, a.w2s_c = (_es(w2, d) for d in range(3))
        keep += [gate, up, w2]
    else:
        (gq, gs), (uq, us), (wq, wsc) = gate_q, up_q, w2_q
        a.I = gq.shape[1]
        for c, s, rows, K in ((gq, gs, a.I, H), (uq, us, a.I, H), (wq, wsc, H, a.I)):
            assert c.dtype == np.uint8 and s.dtype == np.uint8
            assert c.shape == (num_experts, rows, K // 2) and s.shape == (num_experts, rows, K // 32)
            assert c.strides[2] == 1 and s.strides[2] == 1
        a.gate_q, a.up_q, a.w2_q = _ptr(gq), _ptr(uq), _ptr(wq)
        a.gate_sc, a.up_sc, a.w2_sc = _ptr(gs), _ptr(us), _ptr(wsc)
        a.gqs_e, a.gqs_r = gq.strides[0], gq.strides[1]
        a.uqs_e, a.uqs_r = uq.strides[0], uq.strides[1]
        a.w2qs_e, a.w2qs_r = wq.strides[0], wq.strides[1]
        a.gss_e, a.gss_r = gs.strides[0], gs.strides[1]
        a.uss_e, a.uss_r = us.strides[0], us.strides[1]
        a.w2ss_e, a.w2ss_r = wsc.strides[0], wsc.strides[1]
        keep += [gq, gs, uq, us, wq, wsc]
    assert ids.dtype == np.int32 and wts.dtype == np.float32 and ids.shape == wts.shape
    a.ids, a.is_t, a.is_j = _ptr(ids), _es(ids, 0), _es(ids, 1)
    a.wts, a.ws_t, a.ws_j = _ptr(wts), _es(wts, 0), _es(wts, 1)
    if toks is None:
        n = T
        tp = None
    else:
        toks = np.ascontiguousarray(toks, dtype=np.int64)
        n = toks.size
        tp = _ptr(toks)
    out_acc = np.zeros((n, H), dtype=np.float64)
    out_bf16 = np.zeros((n, H), dtype=np.uint16)
    rc = lib().orc_ffn(ctypes.byref(a), tp, n, _ptr(out_acc), _ptr(out_bf16))
    del keep
    if rc != 0:
        raise ValueError("orc_ffn failed")
    return out_acc, out_bf16


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float64 (exact)."""
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- rmsnorm

def rmsnorm(x_bits: np.ndarray, weight: np.ndarray, eps: float) -> tuple[np.ndarray, np.ndarray]:
    """RMSNorm of bf16 bits x [T, H] (any strides) with float64 weight [H]
    (any stride). Returns (float64 [T, H], bf16 bits uint16 [T, H])."""
    assert x_bits.dtype == np.uint16 and x_bits.ndim == 2
    weight = np.asarray(weight, dtype=np.float64)
    T, H = x_bits.shape
    acc = np.empty((T, H), dtype=np.float64)
    bits = np.empty((T, H), dtype=np.uint16)
    rc = lib().orc_rmsnorm(_ptr(x_bits), T, H, _es(x_bits, 0), _es(x_bits, 1), _ptr(weight),
                           _es(weight, 0), float(eps), _ptr(acc), _ptr(bits))
    if rc != 0:
        raise ValueError("orc_rmsnorm failed")
    return acc, bits


# --------------------------------------------------------------- backward

def ffn_bwd(x_bits: np.ndarray, ids: np.ndarray, wts: np.ndarray, dout_bits: np.ndarray, *,
            num_experts: int, gate: np.ndarray, up: np.ndarray, w2: np.ndarray,
            toks: Optional[np.ndarray] = None, exps: Optional[np.ndarray] = None,
            round_h: bool = True):
    """Gradients of sum(dout * out) for the bf16 forward (plain definition).

    x, dout: bf16 bits [T, H] (any strides); gate/up [E, I, H], w2 [E, H, I]
    bf16 bits (any strides). dx/dw for the tokens ``toks`` (all if None), the
    weight gradients for the experts ``exps`` (none if None). Returns
    (dx float64 [n, H], dx bf16 bits [n, H], dw float64 [n, k],
     dgate float64 [m, I, H], dup float64 [m, I, H], dw2 float64 [m, H, I]).
    """
    a = _FfnArgs()
    T, H = x_bits.shape
    assert x_bits.dtype == np.uint16 and dout_bits.dtype == np.uint16 and dout_bits.shape == (T, H)
    a.mode, a.round_h = 0, int(round_h)
    a.T, a.H, a.E, a.k = T, H, num_experts, ids.shape[1]
    a.I = gate.shape[1]
    a.x, a.xs_t, a.xs_h = _ptr(x_bits), _es(x_bits, 0), _es(x_bits, 1)
    a.gate, a.up, a.w2 = _ptr(gate), _ptr(up), _ptr(w2)
    a.gs_e, a.gs_r, a.gs_c = (_es(gate, d) for d in range(3))
    a.us_e, a.us_r, a.us_c = (_es(up, d) for d in range(3))
    a.w2s_e, a.w2s_r, a.w2s_c = (_es(w2, d) for d in range(3))
    assert ids.dtype == np.int32 and wts.dtype == np.float32 and ids.shape == wts.shape
    a.ids, a.is_t, a.is_j = _ptr(ids), _es(ids, 0), _es(ids, 1)
    a.wts, a.ws_t, a.ws_j = _ptr(wts), _es(wts, 0), _es(wts, 1)
    toks = np.arange(T, dtype=np.int64) if toks is None else np.ascontiguousarray(toks, dtype=np.int64)
    exps = np.zeros(0, dtype=np.int64) if exps is None else np.ascontiguousarray(exps, dtype=np.int64)
    n, m, I, k = toks.size, exps.size, a.I, a.k
    dx = np.zeros((n, H))
    dxb = np.zeros((n, H), dtype=np.uint16)
    dw = np.zeros((n, k))
    dg = np.zeros((m, I, H))
    du = np.zeros((m, I, H))
    dw2 = np.zeros((m, H, I))
    keep = [x_bits, ids, wts, dout_bits, gate, up, w2, toks, exps]
    rc = lib().orc_ffn_bwd(ctypes.byref(a), _ptr(dout_bits), _es(dout_bits, 0), _es(dout_bits, 1),
                           _ptr(toks), n, _ptr(dx), _ptr(dxb), _ptr(dw), _ptr(exps), m,
                           _ptr(dg), _ptr(du), _ptr(dw2))
    del keep
    if rc != 0:
        raise ValueError("orc_ffn_bwd failed")
    return dx, dxb, dw, dg, du, dw2
