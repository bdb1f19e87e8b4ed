"""Routed-MoE expert path for one AMD Instinct MI355X (gfx950).

local dispatch -> grouped gate-up GEMM with a fused SiLU-gated epilogue ->
grouped down GEMM -> weighted top-k combine, as hand-written HIP kernels
behind the C ABI in include/moe_mi355x.h (libmoe_mi355x.so).  This package is
the thin Python binding: `ops` marshals torch tensors into that ABI.
"""
from ._lib import (HINT_AUTO, HINT_SKINNY, HINT_TILED64, HINT_TILED128, HINT_TILED_LARGE, LIB_PATH, MoeError,
                   MoeProblem, lib, problem, status_string, workspace_size)
from . import ops

__all__ = [
    "ops", "lib", "problem", "workspace_size", "status_string", "MoeError", "MoeProblem",
    "LIB_PATH", "HINT_AUTO", "HINT_SKINNY", "HINT_TILED64", "HINT_TILED128", "HINT_TILED_LARGE",
]
