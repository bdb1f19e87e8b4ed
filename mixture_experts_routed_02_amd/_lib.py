"""ctypes view of libmoe_mi355x.so (the C ABI in include/moe_mi355x.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Loading fails loudly when the library has not been built; there is
no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

MOE_SUCCESS = 0
MOE_ERROR_INVALID_VALUE = 1
MOE_ERROR_NOT_SUPPORTED = 2
MOE_ERROR_LAUNCH = 3

# kernel_hint values
HINT_AUTO, HINT_SKINNY, HINT_TILED64, HINT_TILED128, HINT_TILED_LARGE = 0, 1, 2, 3, 4

EXPORTS = (
    "moe_status_string", "moe_workspace_size", "moe_dispatch", "moe_expert_compute",
    "moe_gate_up", "moe_down", "moe_combine", "moe_router_topk", "moe_forward", "moe_graph_create",
    "moe_graph_launch", "moe_graph_destroy", "moe_mxfp8_quantize", "moe_mxfp8_dequantize",
    "moe_gate_up_mxfp8", "moe_forward_mxfp8", "moe_mxfp4_quantize", "moe_mxfp4_dequantize",
    "moe_gate_up_mxfp4", "moe_forward_mxfp4", "moe_skinny_pack", "moe_gate_up_packed",
    "moe_forward_packed", "moe_mx_pack", "moe_gate_up_mx_packed", "moe_forward_mx_packed",
    "moe_forward_noalloc", "moe_router_dispatch", "moe_forward_logits", "moe_tiled_pack",
    "moe_gate_up_tiled_packed", "moe_forward_tiled_packed", "moe_forward_single",
    "moe_single_launch_status", "moe_mx_tiled_pack", "moe_gate_up_mx_tiled_packed",
    "moe_forward_mx_tiled_packed",
)

# Largest moe_forward workspace that moe_forward_noalloc serves from its
# library-owned array (bytes).
NOALLOC_MAX_WORKSPACE = 128 << 20


class MoeProblem(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("intermediate", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("kernel_hint", ctypes.c_int32),
    ]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


_P = ctypes.c_void_p
_PP = ctypes.POINTER(MoeProblem)
_SZ = ctypes.c_size_t

_SIGS = {
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_workspace_size": (ctypes.c_int, [_PP, ctypes.POINTER(_SZ)]),
    "moe_dispatch": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_expert_compute": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_gate_up": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P]),
    "moe_down": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P]),
    "moe_combine": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P]),
    "moe_router_topk": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P]),
    "moe_forward": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_graph_create": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                        ctypes.POINTER(ctypes.c_void_p)]),
    "moe_graph_launch": (ctypes.c_int, [_P, _P]),
    "moe_mxfp8_quantize": (ctypes.c_int, [_P, ctypes.c_int64, ctypes.c_int32, _P, _P, _P]),
    "moe_mxfp8_dequantize": (ctypes.c_int, [_P, _P, ctypes.c_int64, ctypes.c_int32, _P, _P]),
    "moe_gate_up_mxfp8": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P]),
    "moe_forward_mxfp8": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_mxfp4_quantize": (ctypes.c_int, [_P, ctypes.c_int64, ctypes.c_int32, _P, _P, _P]),
    "moe_skinny_pack": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, _P, _P]),
    "moe_gate_up_packed": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P]),
    "moe_mx_pack": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_int32, _P, _P]),
    "moe_gate_up_mx_packed": (ctypes.c_int, [_PP, ctypes.c_int32, _P, _P, _P, _P, _P, _P]),
    "moe_forward_mx_packed": (ctypes.c_int, [_PP, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P,
                                             _P, _P, _P, _SZ, _P]),
    "moe_forward_packed": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_mxfp4_dequantize": (ctypes.c_int, [_P, _P, ctypes.c_int64, ctypes.c_int32, _P, _P]),
    "moe_gate_up_mxfp4": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P]),
    "moe_forward_mxfp4": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_graph_destroy": (ctypes.c_int, [_P]),
    "moe_forward_noalloc": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_router_dispatch": (ctypes.c_int, [_PP, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P,
                                           _P, _P, _SZ, _P]),
    "moe_forward_logits": (ctypes.c_int, [_PP, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P,
                                          _P, _P, _SZ, _P]),
    "moe_tiled_pack": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P]),
    "moe_gate_up_tiled_packed": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P]),
    "moe_forward_tiled_packed": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_forward_single": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_single_launch_status": (ctypes.c_int, [ctypes.POINTER(ctypes.c_uint32)]),
    "moe_mx_tiled_pack": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, _P, _P]),
    "moe_gate_up_mx_tiled_packed": (ctypes.c_int, [_PP, ctypes.c_int32, _P, _P, _P, _P, _P, _P]),
    "moe_forward_mx_tiled_packed": (ctypes.c_int, [_PP, ctypes.c_int32, _P, _P, _P, _P, _P, _P,
                                                   _P, _P, _P, _P, _P, _SZ, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once).  Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m mixture_experts_routed_02_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def check(fn: str, status: int) -> None:
    if status != MOE_SUCCESS:
        raise MoeError(fn, status, status_string(status))


def problem(num_tokens, top_k, num_experts, hidden, intermediate, capacity=0, kernel_hint=0):
    return MoeProblem(int(num_tokens), int(top_k), int(num_experts), int(hidden),
                      int(intermediate), int(capacity), int(kernel_hint))


def workspace_size(p: MoeProblem) -> int:
    n = _SZ(0)
    check("moe_workspace_size", lib().moe_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return int(n.value)
