"""ctypes mirror of include/moeffn.h and the library loader.

The library is loaded from this package directory only. If it is missing the
import of a compute entry point raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoeffn.so")

MOE_MAX_DIMS = 4
MOE_NUM_STAGES = 5

DT_BF16, DT_F32, DT_I32, DT_FP4X2, DT_E8M0 = 1, 2, 3, 4, 5
MODE_BF16, MODE_MXFP4 = 0, 1
ACT_SILU = 0

STATUS = {0: "MOE_OK", -1: "MOE_ERR_NULL", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_DTYPE",
          -4: "MOE_ERR_LAYOUT", -5: "MOE_ERR_WORKSPACE", -6: "MOE_ERR_UNSUPPORTED",
          -7: "MOE_ERR_HIP", -8: "MOE_ERR_ARG"}
STAGES = ("align", "prepare", "gemm1", "gemm2", "combine")


class TensorDesc(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("size", ctypes.c_int64 * MOE_MAX_DIMS), ("stride", ctypes.c_int64 * MOE_MAX_DIMS)]


class FusedArgs(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("activation", ctypes.c_int32),
                ("x", TensorDesc), ("gate", TensorDesc), ("up", TensorDesc),
                ("gate_scale", TensorDesc), ("up_scale", TensorDesc),
                ("w2", TensorDesc), ("w2_scale", TensorDesc),
                ("topk_ids", TensorDesc), ("topk_weights", TensorDesc), ("out", TensorDesc),
                ("stage_events", ctypes.c_void_p), ("force_config", ctypes.c_int32),
                ("expert_offset", ctypes.c_int32), ("y_rows", TensorDesc),
                ("num_global_experts", ctypes.c_int32), ("norm_eps", ctypes.c_float),
                ("norm_weight", TensorDesc)]


class BwdArgs(ctypes.Structure):
    _fields_ = [("fwd", FusedArgs), ("dout", TensorDesc), ("dx", TensorDesc), ("dgate", TensorDesc),
                ("dup", TensorDesc), ("dw2", TensorDesc), ("dtopk_weights", TensorDesc),
                ("accumulate", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class Config(ctypes.Structure):
    _fields_ = [("bucket", ctypes.c_int32), ("block_m", ctypes.c_int32),
                ("gemm1_kernel", ctypes.c_int32), ("gemm2_kernel", ctypes.c_int32),
                ("gemm1_split_k", ctypes.c_int32), ("gemm2_split_k", ctypes.c_int32),
                ("config_index", ctypes.c_int32), ("num_configs", ctypes.c_int32),
                ("block_m2", ctypes.c_int32)]


EXPORTS = ("moe_topk_softmax", "moe_align", "moe_align_capacity", "moe_align_workspace_size",
           "moe_quant_mxfp4", "moe_query_config", "moe_fused_workspace_size", "moe_fused_fwd",
           "moe_fused_fwd_noalloc",
           "moe_combine", "moe_rmsnorm", "moe_fused_bwd_workspace_size", "moe_fused_bwd",
           "moe_strerror", "moe_last_error")

_lib = None


class MoEError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


def load() -> ctypes.CDLL:
    """Load libmoeffn.so (built in-tree by build.build()); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run mixture_experts_ffn_align_amd.build.build()")
    L = ctypes.CDLL(LIB_PATH)
    P, vp, i32, i64 = ctypes.POINTER, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    TD = P(TensorDesc)
    L.moe_topk_softmax.argtypes = [TD, i32, i32, i32, ctypes.c_float, TD, TD, vp]
    L.moe_align.argtypes = [TD, i32, i32, TD, TD, TD, vp, ctypes.c_size_t, vp]
    L.moe_align_capacity.argtypes = [i64, i32, i32]
    L.moe_align_capacity.restype = i64
    L.moe_align_workspace_size.argtypes = [i64, i32, i32, i32, P(ctypes.c_size_t)]
    L.moe_quant_mxfp4.argtypes = [TD, TD, TD, vp]
    L.moe_query_config.argtypes = [P(FusedArgs), P(Config)]
    L.moe_fused_workspace_size.argtypes = [P(FusedArgs), P(ctypes.c_size_t)]
    L.moe_fused_fwd.argtypes = [P(FusedArgs), vp, ctypes.c_size_t, vp]
    L.moe_fused_fwd_noalloc.argtypes = [P(FusedArgs), vp]
    L.moe_combine.argtypes = [TD, TD, TD, i32, TD, vp]
    L.moe_rmsnorm.argtypes = [TD, TD, ctypes.c_float, TD, vp]
    L.moe_fused_bwd_workspace_size.argtypes = [P(BwdArgs), P(ctypes.c_size_t)]
    L.moe_fused_bwd.argtypes = [P(BwdArgs), vp, ctypes.c_size_t, vp]
    L.moe_strerror.argtypes = [ctypes.c_int]
    L.moe_strerror.restype = ctypes.c_char_p
    L.moe_last_error.restype = ctypes.c_char_p
    for name in ("moe_topk_softmax", "moe_align", "moe_align_workspace_size", "moe_quant_mxfp4",
                 "moe_query_config", "moe_fused_workspace_size", "moe_fused_fwd", "moe_fused_fwd_noalloc",
                 "moe_combine",
                 "moe_rmsnorm", "moe_fused_bwd_workspace_size", "moe_fused_bwd"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def check(status: int) -> None:
    if status != 0:
        detail = load().moe_last_error().decode()
        raise MoEError(status, detail)
