"""ctypes loader for libmoe_mi355x.so and the signatures of its C ABI.

The library is loaded on first use.  If it is missing, every call raises:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355x.so")

MOE_F32, MOE_BF16 = 0, 1
ROUTE_MODES = {"softmax": 0, "gumbel": 1}
ACTS = {"swiglu": 0, "gelu": 1}
MAX_EXPERTS = 64
MAX_TOPK = 8

STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_DTYPE",
                4: "MOE_ERR_UNSUPPORTED", 5: "MOE_ERR_ALIGN", 6: "MOE_ERR_WORKSPACE",
                7: "MOE_ERR_LAUNCH"}

# Every symbol include/moe.h declares.
EXPORTS = ("moe_capacity", "moe_status_string", "moe_workspace_bytes", "moe_route",
           "moe_aux_stats", "moe_dispatch", "moe_expert_ffn", "moe_expert_ffn_gather",
           "moe_expert_ffn_ws_bytes", "moe_combine", "moe_combine_bwd", "moe_expert_ffn_bwd",
           "moe_expert_ffn_bwd_ws_bytes", "moe_dispatch_bwd", "moe_route_bwd",
           "moe_route_bwd_ws_bytes", "moe_quantize_fp8", "moe_dequantize_fp8",
           "moe_expert_ffn_fp8", "moe_expert_ffn_gather_fp8", "moe_expert_ffn_fwd_save",
           "moe_dispatch_aux", "moe_dispatch_aux_noalloc", "moe_expert_ffn_gather_combine",
           "moe_expert_ffn_combine_ws_bytes", "moe_expert_ffn_gather_combine_fp8")

_lock = threading.Lock()
_lib = None


class MoEError(RuntimeError):
    """A non-zero status from the C ABI."""

    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)} ({text})")
        self.status = status


def _declare(L: ctypes.CDLL) -> None:
    c = ctypes
    vp, i32, i64, u64, f32, f64 = c.c_void_p, c.c_int, c.c_int64, c.c_uint64, c.c_float, c.c_double
    L.moe_capacity.argtypes = [i64, i32, i32, f64]
    L.moe_capacity.restype = i64
    L.moe_status_string.argtypes = [i32]
    L.moe_status_string.restype = c.c_char_p
    L.moe_workspace_bytes.argtypes = [i64, i32, i32]
    L.moe_workspace_bytes.restype = c.c_size_t
    L.moe_route.argtypes = [vp, i32, vp, vp, vp, i64, i64, i32, i32, i32, u64, i64,
                            vp, vp, vp, vp]
    L.moe_route.restype = i32
    L.moe_aux_stats.argtypes = [vp, vp, vp, i64, i32, i32, f32, vp, vp, vp, vp, vp, c.c_size_t]
    L.moe_aux_stats.restype = i32
    L.moe_dispatch.argtypes = [vp, i32, vp, vp, i64, i64, i32, i32, i64, vp, vp, vp, vp, vp,
                               vp, c.c_size_t]
    L.moe_dispatch.restype = i32
    L.moe_dispatch_aux.argtypes = [vp, i32, vp, vp, vp, i64, i64, i32, i32, i64, f32, vp, vp, vp,
                                   vp, vp, vp, vp, vp, vp, vp, c.c_size_t]
    L.moe_dispatch_aux.restype = i32
    L.moe_dispatch_aux_noalloc.argtypes = [vp, i32, vp, vp, vp, i64, i64, i32, i32, i64, f32, vp,
                                           vp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_dispatch_aux_noalloc.restype = i32
    L.moe_expert_ffn.argtypes = [vp, i32, i32, vp, vp, i32, i64, i64, i64, vp, vp, vp, vp, vp,
                                 vp, vp, vp, c.c_size_t]
    L.moe_expert_ffn.restype = i32
    L.moe_expert_ffn_gather.argtypes = [vp, i32, i32, vp, vp, i64, vp, i32, i64, i64, i64, vp,
                                        vp, vp, vp, vp, vp, vp, vp, c.c_size_t]
    L.moe_expert_ffn_gather.restype = i32
    L.moe_expert_ffn_ws_bytes.argtypes = []
    L.moe_expert_ffn_ws_bytes.restype = c.c_size_t
    L.moe_combine.argtypes = [vp, i32, vp, vp, vp, i64, i64, i32, vp, vp]
    L.moe_combine.restype = i32
    L.moe_combine_bwd.argtypes = [vp, i32, vp, vp, vp, vp, i64, i64, i32, vp, vp]
    L.moe_combine_bwd.restype = i32
    L.moe_expert_ffn_bwd.argtypes = [vp, i32, i32, vp, vp, i32, i64, i64, i64, vp, vp, vp, vp, vp,
                                     vp, vp, vp, vp, vp, vp, vp, c.c_size_t, i32]
    L.moe_expert_ffn_fwd_save.argtypes = [vp, i32, i32, vp, vp, i32, i64, i64, i64, vp, vp, vp,
                                          vp, vp, vp, vp, c.c_size_t]
    L.moe_expert_ffn_fwd_save.restype = i32
    L.moe_expert_ffn_bwd.restype = i32
    L.moe_expert_ffn_bwd_ws_bytes.argtypes = [i32, i64, i64]
    L.moe_expert_ffn_bwd_ws_bytes.restype = c.c_size_t
    L.moe_dispatch_bwd.argtypes = [vp, vp, vp, i64, i64, i32, vp, vp]
    L.moe_dispatch_bwd.restype = i32
    L.moe_route_bwd.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, f32, f32, i64, i64, i32,
                                i32, i64, vp, vp, vp, vp, vp, c.c_size_t]
    L.moe_route_bwd.restype = i32
    L.moe_route_bwd_ws_bytes.argtypes = [i64, i64, i32]
    L.moe_route_bwd_ws_bytes.restype = c.c_size_t
    L.moe_quantize_fp8.argtypes = [vp, vp, i32, i64, i64, vp, vp]
    L.moe_quantize_fp8.restype = i32
    L.moe_dequantize_fp8.argtypes = [vp, vp, vp, i32, i64, i64, vp]
    L.moe_dequantize_fp8.restype = i32
    L.moe_expert_ffn_fp8.argtypes = [vp, i32, vp, vp, i32, i64, i64, i64, vp, vp, vp, vp, vp, vp,
                                     vp, vp, vp, vp, vp, c.c_size_t]
    L.moe_expert_ffn_fp8.restype = i32
    L.moe_expert_ffn_gather_fp8.argtypes = [vp, i32, vp, vp, i64, vp, i32, i64, i64, i64, vp, vp,
                                            vp, vp, vp, vp, vp, vp, vp, vp, vp, c.c_size_t]
    L.moe_expert_ffn_gather_fp8.restype = i32
    L.moe_expert_ffn_gather_combine.argtypes = [vp, i32, vp, vp, vp, vp, i64, i32, vp, i32, i64,
                                                i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                c.c_size_t, vp]
    L.moe_expert_ffn_gather_combine.restype = i32
    L.moe_expert_ffn_gather_combine_fp8.argtypes = [vp, i32, vp, vp, vp, vp, i64, i32, vp, i32,
                                                    i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                                    vp, vp, vp, vp, c.c_size_t, vp]
    L.moe_expert_ffn_gather_combine_fp8.restype = i32
    L.moe_expert_ffn_combine_ws_bytes.argtypes = [i64, i64]
    L.moe_expert_ffn_combine_ws_bytes.restype = c.c_size_t


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m mixture_experts_layer_08_amd.build` (there is no fallback)")
            L = ctypes.CDLL(LIB_PATH)
            _declare(L)
            _lib = L
    return _lib


def check(fn: str, status: int) -> None:
    if status != 0:
        text = lib().moe_status_string(status).decode()
        raise MoEError(fn, status, text)
