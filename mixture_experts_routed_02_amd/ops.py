"""Thin torch-tensor wrappers over the C ABI (argument marshalling only).

PyTorch provides device memory and the current HIP stream; every step of the
layer runs in libmoe_mi355x.so.  Each wrapper checks dtypes, shapes and
devices, passes raw pointers and the stream, and raises MoeError on a
non-success status.  Nothing here computes any part of the layer.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import MoeProblem, check, lib, problem, workspace_size

__all__ = [
    "problem", "workspace_size", "make_workspace", "dispatch", "expert_compute", "gate_up",
    "down", "combine",
    "forward", "MoEGraph", "MoeProblem", "mx_quantize", "mx_dequantize", "gate_up_mx", "forward_mx",
    "mxfp8_quantize", "mxfp8_dequantize", "gate_up_mxfp8", "forward_mxfp8", "skinny_pack",
    "gate_up_packed", "forward_packed", "mx_pack", "forward_noalloc", "router_dispatch",
    "forward_logits", "tiled_pack", "gate_up_tiled_packed", "forward_tiled_packed",
    "forward_single", "single_launch_status", "mx_tiled_pack",
]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _cap(p: MoeProblem) -> int:
    return p.capacity or p.num_tokens * p.top_k


def make_workspace(p: MoeProblem, device) -> torch.Tensor:
    """Device workspace for every entry point of problem p (uint8, 256-B aligned)."""
    n = workspace_size(p)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _ntok(num_tokens_dev, device):
    if num_tokens_dev is None:
        return None
    _need(num_tokens_dev, "num_tokens_dev", torch.int32, (1,), device)
    return num_tokens_dev


def dispatch(p: MoeProblem, x, topk_ids, num_tokens_dev=None, workspace=None, out=None):
    """Local dispatch.  Returns (x_disp [cap,H], expert_offsets [E+1], row_src [cap],
    token_row [T*K])."""
    T, K, E, H = p.num_tokens, p.top_k, p.num_experts, p.hidden
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, H))
    _need(topk_ids, "topk_ids", torch.int32, (T, K), dev)
    nt = _ntok(num_tokens_dev, dev)
    cap = _cap(p)
    if out is None:
        out = (torch.empty((cap, H), dtype=torch.bfloat16, device=dev),
               torch.empty((E + 1,), dtype=torch.int32, device=dev),
               torch.empty((max(cap, 1),), dtype=torch.int32, device=dev),
               torch.empty((max(T * K, 1),), dtype=torch.int32, device=dev))
    x_disp, offsets, row_src, token_row = out
    ws = make_workspace(p, dev) if workspace is None else workspace
    check("moe_dispatch", lib().moe_dispatch(
        ctypes.byref(p), _ptr(x), _ptr(topk_ids), _ptr(nt), _ptr(x_disp), _ptr(offsets),
        _ptr(row_src), _ptr(token_row), _ptr(ws), ws.numel(), _stream_ptr(dev)))
    return x_disp, offsets, row_src, token_row


def expert_compute(p: MoeProblem, x_disp, expert_offsets, w_gateup, w_down, workspace=None,
                   y_disp=None):
    """Dispatched-expert MLP over a tight expert-major batch.  Returns y_disp [cap, H]."""
    E, H, I = p.num_experts, p.hidden, p.intermediate
    dev = x_disp.device
    cap = _cap(p)
    _need(x_disp, "x_disp", torch.bfloat16, (cap, H))
    _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,), dev)
    _need(w_gateup, "w_gateup", torch.bfloat16, (E, 2 * I, H), dev)
    _need(w_down, "w_down", torch.bfloat16, (E, H, I), dev)
    if y_disp is None:
        y_disp = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
    _need(y_disp, "y_disp", torch.bfloat16, (cap, H), dev)
    ws = make_workspace(p, dev) if workspace is None else workspace
    check("moe_expert_compute", lib().moe_expert_compute(
        ctypes.byref(p), _ptr(x_disp), _ptr(expert_offsets), _ptr(w_gateup), _ptr(w_down),
        _ptr(y_disp), _ptr(ws), ws.numel(), _stream_ptr(dev)))
    return y_disp


def gate_up(p: MoeProblem, x_disp, expert_offsets, w_gateup, h=None):
    """Gate-up grouped GEMM with the SiLU-gated epilogue.  Returns h [cap, I]."""
    E, H, I = p.num_experts, p.hidden, p.intermediate
    dev = x_disp.device
    cap = _cap(p)
    _need(x_disp, "x_disp", torch.bfloat16, (cap, H))
    _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,), dev)
    _need(w_gateup, "w_gateup", torch.bfloat16, (E, 2 * I, H), dev)
    if h is None:
        h = torch.empty((cap, I), dtype=torch.bfloat16, device=dev)
    _need(h, "h", torch.bfloat16, (cap, I), dev)
    check("moe_gate_up", lib().moe_gate_up(ctypes.byref(p), _ptr(x_disp), _ptr(expert_offsets),
                                           _ptr(w_gateup), _ptr(h), _stream_ptr(dev)))
    return h


def down(p: MoeProblem, h, expert_offsets, w_down, y_disp=None):
    """Down grouped GEMM.  Returns y_disp [cap, H]."""
    E, H, I = p.num_experts, p.hidden, p.intermediate
    dev = h.device
    cap = _cap(p)
    _need(h, "h", torch.bfloat16, (cap, I))
    _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,), dev)
    _need(w_down, "w_down", torch.bfloat16, (E, H, I), dev)
    if y_disp is None:
        y_disp = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
    _need(y_disp, "y_disp", torch.bfloat16, (cap, H), dev)
    check("moe_down", lib().moe_down(ctypes.byref(p), _ptr(h), _ptr(expert_offsets),
                                     _ptr(w_down), _ptr(y_disp), _stream_ptr(dev)))
    return y_disp


def combine(p: MoeProblem, y_disp, token_row, topk_weights, num_tokens_dev=None, out=None):
    """Weighted top-k combine.  Returns out [T, H] (rows t >= T_v untouched)."""
    T, K, H = p.num_tokens, p.top_k, p.hidden
    dev = y_disp.device
    _need(y_disp, "y_disp", torch.bfloat16, (_cap(p), H))
    _need(token_row, "token_row", torch.int32, None, dev)
    if token_row.numel() < T * K:
        raise ValueError("token_row must hold T*K entries")
    _need(topk_weights, "topk_weights", torch.float32, (T, K), dev)
    nt = _ntok(num_tokens_dev, dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (T, H), dev)
    check("moe_combine", lib().moe_combine(
        ctypes.byref(p), _ptr(y_disp), _ptr(token_row), _ptr(topk_weights), _ptr(nt), _ptr(out),
        _stream_ptr(dev)))
    return out


def router_topk(p: MoeProblem, logits, num_tokens_dev=None, topk_ids=None, topk_weights=None):
    """Router top-k over fp32 logits [T, E]: the K largest per token (equal
    values in increasing expert index) and the softmax over them.  Returns
    (topk_ids int32 [T, K], topk_weights fp32 [T, K]); rows t >= T_v are left
    as they were."""
    T, K, E = p.num_tokens, p.top_k, p.num_experts
    dev = logits.device
    _need(logits, "logits", torch.float32, (T, E))
    nt = _ntok(num_tokens_dev, dev)
    if topk_ids is None:
        topk_ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    if topk_weights is None:
        topk_weights = torch.empty((T, K), dtype=torch.float32, device=dev)
    _need(topk_ids, "topk_ids", torch.int32, (T, K), dev)
    _need(topk_weights, "topk_weights", torch.float32, (T, K), dev)
    check("moe_router_topk", lib().moe_router_topk(
        ctypes.byref(p), _ptr(logits), _ptr(nt), _ptr(topk_ids), _ptr(topk_weights),
        _stream_ptr(dev)))
    return topk_ids, topk_weights


def _routing_outs(p, logits, topk_ids, topk_weights):
    T, K = p.num_tokens, p.top_k
    dev = logits.device
    _need(logits, "logits", torch.float32)
    if logits.dim() != 2 or logits.shape[0] != T:
        raise ValueError(f"logits must be [{T}, router_experts], got {tuple(logits.shape)}")
    if topk_ids is None:
        topk_ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    if topk_weights is None:
        topk_weights = torch.empty((T, K), dtype=torch.float32, device=dev)
    _need(topk_ids, "topk_ids", torch.int32, (T, K), dev)
    _need(topk_weights, "topk_weights", torch.float32, (T, K), dev)
    return topk_ids, topk_weights


def router_dispatch(p: MoeProblem, logits, x, num_tokens_dev=None, topk_ids=None,
                    topk_weights=None, workspace=None, out=None):
    """The router step fused ahead of dispatch, from fp32 logits [T, G] (G router
    experts; ids >= num_experts are dropped as non-local).  Returns (topk_ids,
    topk_weights, x_disp, expert_offsets, row_src, token_row)."""
    T, K, E, H = p.num_tokens, p.top_k, p.num_experts, p.hidden
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, H), dev)
    topk_ids, topk_weights = _routing_outs(p, logits, topk_ids, topk_weights)
    nt = _ntok(num_tokens_dev, dev)
    cap = _cap(p)
    if out is None:
        out = (torch.empty((cap, H), dtype=torch.bfloat16, device=dev),
               torch.empty((E + 1,), dtype=torch.int32, device=dev),
               torch.empty((max(cap, 1),), dtype=torch.int32, device=dev),
               torch.empty((max(T * K, 1),), dtype=torch.int32, device=dev))
    x_disp, offsets, row_src, token_row = out
    ws = make_workspace(p, dev) if workspace is None else workspace
    check("moe_router_dispatch", lib().moe_router_dispatch(
        ctypes.byref(p), int(logits.shape[1]), _ptr(logits), _ptr(nt), _ptr(topk_ids),
        _ptr(topk_weights), _ptr(x), _ptr(x_disp), _ptr(offsets), _ptr(row_src), _ptr(token_row),
        _ptr(ws), ws.numel(), _stream_ptr(dev)))
    return topk_ids, topk_weights, x_disp, offsets, row_src, token_row


def forward_logits(p: MoeProblem, logits, x, w_gateup, w_down, num_tokens_dev=None,
                   topk_ids=None, topk_weights=None, expert_offsets=None, out=None,
                   workspace=None):
    """The whole layer from router logits [T, G] (router fused into dispatch).
    Returns (out [T,H], expert_offsets [E+1], topk_ids, topk_weights)."""
    topk_ids, topk_weights = _routing_outs(p, logits, topk_ids, topk_weights)
    nt, offsets, out, ws = _forward_args(p, x, topk_ids, topk_weights, w_gateup, w_down,
                                         num_tokens_dev, expert_offsets, out, workspace)
    check("moe_forward_logits", lib().moe_forward_logits(
        ctypes.byref(p), int(logits.shape[1]), _ptr(logits), _ptr(x), _ptr(w_gateup),
        _ptr(w_down), _ptr(nt), _ptr(topk_ids), _ptr(topk_weights), _ptr(offsets), _ptr(out),
        _ptr(ws), ws.numel(), _stream_ptr(x.device)))
    return out, offsets, topk_ids, topk_weights


def _forward_args(p, x, topk_ids, topk_weights, w_gateup, w_down, num_tokens_dev, offsets, out,
                  workspace):
    T, K, E, H, I = p.num_tokens, p.top_k, p.num_experts, p.hidden, p.intermediate
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, H))
    _need(topk_ids, "topk_ids", torch.int32, (T, K), dev)
    _need(topk_weights, "topk_weights", torch.float32, (T, K), dev)
    _need(w_gateup, "w_gateup", torch.bfloat16, (E, 2 * I, H), dev)
    _need(w_down, "w_down", torch.bfloat16, (E, H, I), dev)
    nt = _ntok(num_tokens_dev, dev)
    if offsets is None:
        offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    _need(offsets, "expert_offsets", torch.int32, (E + 1,), dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (T, H), dev)
    if workspace is False:      # the caller passes no workspace
        return nt, offsets, out, None
    ws = make_workspace(p, dev) if workspace is None else workspace
    return nt, offsets, out, ws


def forward(p: MoeProblem, x, topk_ids, topk_weights, w_gateup, w_down, num_tokens_dev=None,
            expert_offsets=None, out=None, workspace=None):
    """The whole routed-expert layer.  Returns (out [T,H], expert_offsets [E+1])."""
    nt, offsets, out, ws = _forward_args(p, x, topk_ids, topk_weights, w_gateup, w_down,
                                         num_tokens_dev, expert_offsets, out, workspace)
    check("moe_forward", lib().moe_forward(
        ctypes.byref(p), _ptr(x), _ptr(topk_ids), _ptr(topk_weights), _ptr(w_gateup),
        _ptr(w_down), _ptr(nt), _ptr(offsets), _ptr(out), _ptr(ws), ws.numel(),
        _stream_ptr(x.device)))
    return out, offsets


def forward_single(p: MoeProblem, x, topk_ids, topk_weights, w_gateup, w_down,
                   num_tokens_dev=None, expert_offsets=None, out=None, workspace=None):
    """The whole layer in one cooperative launch (tiny batches: T*K <= 8,
    I % 1024 == 0).  Returns (out [T,H], expert_offsets [E+1])."""
    nt, offsets, out, ws = _forward_args(p, x, topk_ids, topk_weights, w_gateup, w_down,
                                         num_tokens_dev, expert_offsets, out, workspace)
    check("moe_forward_single", lib().moe_forward_single(
        ctypes.byref(p), _ptr(x), _ptr(topk_ids), _ptr(topk_weights), _ptr(w_gateup),
        _ptr(w_down), _ptr(nt), _ptr(offsets), _ptr(out), _ptr(ws), ws.numel(),
        _stream_ptr(x.device)))
    return out, offsets


def single_launch_status() -> int:
    """Barrier timeouts of forward_single launches on the current device since
    the last call (host-synchronous; resets the barrier state)."""
    n = ctypes.c_uint32(0)
    check("moe_single_launch_status", lib().moe_single_launch_status(ctypes.byref(n)))
    return int(n.value)


def forward_noalloc(p: MoeProblem, x, topk_ids, topk_weights, w_gateup, w_down,
                    num_tokens_dev=None, expert_offsets=None, out=None):
    """moe_forward with the library's own device array as workspace (no
    allocation by the library; at most NOALLOC_MAX_WORKSPACE bytes of
    workspace).  Returns (out [T,H], expert_offsets [E+1])."""
    nt, offsets, out, _ = _forward_args(p, x, topk_ids, topk_weights, w_gateup, w_down,
                                        num_tokens_dev, expert_offsets, out, workspace=False)
    check("moe_forward_noalloc", lib().moe_forward_noalloc(
        ctypes.byref(p), _ptr(x), _ptr(topk_ids), _ptr(topk_weights), _ptr(w_gateup),
        _ptr(w_down), _ptr(nt), _ptr(offsets), _ptr(out), _stream_ptr(x.device)))
    return out, offsets


# ---------------------------------------------------------------------------
# bf16 expert weights in the skinny pack layout (include/moe_mi355x.h)
# ---------------------------------------------------------------------------
def skinny_pack(w, gated: bool, out=None):
    """Pack bf16 weights [E, rows, K] for the skinny kernels (gated: W_gateup)."""
    _need(w, "w", torch.bfloat16)
    if w.dim() != 3:
        raise ValueError("w must be [experts, rows, k]")
    E, rows, K = w.shape
    if out is None:
        out = torch.empty_like(w)
    _need(out, "out", torch.bfloat16, tuple(w.shape), w.device)
    check("moe_skinny_pack", lib().moe_skinny_pack(_ptr(w), E, rows, K, int(bool(gated)), _ptr(out),
                                                   _stream_ptr(w.device)))
    return out


def tiled_pack(w, out=None):
    """Pack bf16 weights [E, rows, K] for the tiled kernels (W_gateup or W_down)."""
    _need(w, "w", torch.bfloat16)
    if w.dim() != 3:
        raise ValueError("w must be [experts, rows, k]")
    E, rows, K = w.shape
    if out is None:
        out = torch.empty_like(w)
    _need(out, "out", torch.bfloat16, tuple(w.shape), w.device)
    check("moe_tiled_pack", lib().moe_tiled_pack(_ptr(w), E, rows, K, _ptr(out),
                                                 _stream_ptr(w.device)))
    return out


def gate_up_tiled_packed(p: MoeProblem, x_disp, expert_offsets, w_gateup_packed, h=None):
    """Gate-up grouped GEMM on weights in the tiled pack layout.  Returns h [cap, I]."""
    E, H, I = p.num_experts, p.hidden, p.intermediate
    dev = x_disp.device
    cap = _cap(p)
    _need(x_disp, "x_disp", torch.bfloat16, (cap, H))
    _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,), dev)
    _need(w_gateup_packed, "w_gateup_packed", torch.bfloat16, (E, 2 * I, H), dev)
    if h is None:
        h = torch.empty((cap, I), dtype=torch.bfloat16, device=dev)
    _need(h, "h", torch.bfloat16, (cap, I), dev)
    check("moe_gate_up_tiled_packed", lib().moe_gate_up_tiled_packed(
        ctypes.byref(p), _ptr(x_disp), _ptr(expert_offsets), _ptr(w_gateup_packed), _ptr(h),
        _stream_ptr(dev)))
    return h


def forward_tiled_packed(p: MoeProblem, x, topk_ids, topk_weights, w_gateup_packed,
                         w_down_packed, num_tokens_dev=None, expert_offsets=None, out=None,
                         workspace=None):
    """The routed-expert layer on weights in the tiled pack layout (tiled plans).
    Returns (out, expert_offsets)."""
    nt, offsets, out, ws = _forward_args(p, x, topk_ids, topk_weights, w_gateup_packed,
                                         w_down_packed, num_tokens_dev, expert_offsets, out,
                                         workspace)
    check("moe_forward_tiled_packed", lib().moe_forward_tiled_packed(
        ctypes.byref(p), _ptr(x), _ptr(topk_ids), _ptr(topk_weights), _ptr(w_gateup_packed),
        _ptr(w_down_packed), _ptr(nt), _ptr(offsets), _ptr(out), _ptr(ws), ws.numel(),
        _stream_ptr(x.device)))
    return out, offsets


def gate_up_packed(p: MoeProblem, x_disp, expert_offsets, w_gateup_packed, h=None):
    """Gate-up grouped GEMM on packed weights.  Returns h [cap, I]."""
    E, H, I = p.num_experts, p.hidden, p.intermediate
    dev = x_disp.device
    cap = _cap(p)
    _need(x_disp, "x_disp", torch.bfloat16, (cap, H))
    _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,), dev)
    _need(w_gateup_packed, "w_gateup_packed", torch.bfloat16, (E, 2 * I, H), dev)
    if h is None:
        h = torch.empty((cap, I), dtype=torch.bfloat16, device=dev)
    _need(h, "h", torch.bfloat16, (cap, I), dev)
    check("moe_gate_up_packed", lib().moe_gate_up_packed(
        ctypes.byref(p), _ptr(x_disp), _ptr(expert_offsets), _ptr(w_gateup_packed), _ptr(h),
        _stream_ptr(dev)))
    return h


def forward_packed(p: MoeProblem, x, topk_ids, topk_weights, w_gateup_packed, w_down_packed,
                   num_tokens_dev=None, expert_offsets=None, out=None, workspace=None):
    """The routed-expert layer on packed bf16 weights.  Returns (out, expert_offsets)."""
    nt, offsets, out, ws = _forward_args(p, x, topk_ids, topk_weights, w_gateup_packed,
                                         w_down_packed, num_tokens_dev, expert_offsets, out,
                                         workspace)
    check("moe_forward_packed", lib().moe_forward_packed(
        ctypes.byref(p), _ptr(x), _ptr(topk_ids), _ptr(topk_weights), _ptr(w_gateup_packed),
        _ptr(w_down_packed), _ptr(nt), _ptr(offsets), _ptr(out), _ptr(ws), ws.numel(),
        _stream_ptr(x.device)))
    return out, offsets


# ---------------------------------------------------------------------------
# MX expert weights (include/moe_mi355x.h): "mxfp8" = e4m3 codes uint8
# [..., K], "mxfp4" = e2m1 codes two per byte uint8 [..., K/2]; both with e8m0
# scales uint8 [..., K/32]
# ---------------------------------------------------------------------------
_MX = {"mxfp8": (8, "mxfp8"), "mxfp4": (4, "mxfp4")}


def _mx(fmt):
    if fmt not in _MX:
        raise ValueError(f"fmt must be one of {sorted(_MX)}")
    return _MX[fmt]


def _mx_code_cols(K, bits):
    return K * bits // 8


def mx_quantize(w, fmt="mxfp8", codes=None, scales=None):
    """Quantize bf16 weights [..., K] (K % 32 == 0) along K.  Returns (codes, scales)."""
    bits_, name = _mx(fmt)
    if not isinstance(w, torch.Tensor) or w.dim() < 1:
        raise TypeError("w must be a torch.Tensor with at least one dimension")
    _need(w, "w", torch.bfloat16)
    K = w.shape[-1]
    if K % 32:
        raise ValueError("the last dimension must be a multiple of 32")
    rows = w.numel() // K if K else 0
    cshape = tuple(w.shape[:-1]) + (_mx_code_cols(K, bits_),)
    sshape = tuple(w.shape[:-1]) + (K // 32,)
    if codes is None:
        codes = torch.empty(cshape, dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty(sshape, dtype=torch.uint8, device=w.device)
    _need(codes, "codes", torch.uint8, cshape, w.device)
    _need(scales, "scales", torch.uint8, sshape, w.device)
    fn = f"moe_{name}_quantize"
    check(fn, getattr(lib(), fn)(_ptr(w), rows, K, _ptr(codes), _ptr(scales), _stream_ptr(w.device)))
    return codes, scales


def mx_dequantize(codes, scales, fmt="mxfp8", out=None):
    """bf16 values of MX weights (the conversion the expert kernels use)."""
    bits_, name = _mx(fmt)
    _need(codes, "codes", torch.uint8)
    K = codes.shape[-1] * 8 // bits_
    _need(scales, "scales", torch.uint8, tuple(codes.shape[:-1]) + (K // 32,), codes.device)
    oshape = tuple(codes.shape[:-1]) + (K,)
    if out is None:
        out = torch.empty(oshape, dtype=torch.bfloat16, device=codes.device)
    _need(out, "out", torch.bfloat16, oshape, codes.device)
    rows = codes.numel() // codes.shape[-1] if codes.shape[-1] else 0
    fn = f"moe_{name}_dequantize"
    check(fn, getattr(lib(), fn)(_ptr(codes), _ptr(scales), rows, K, _ptr(out),
                                 _stream_ptr(codes.device)))
    return out


def mxfp8_quantize(w, codes=None, scales=None):
    return mx_quantize(w, "mxfp8", codes, scales)


def mxfp8_dequantize(codes, scales, out=None):
    return mx_dequantize(codes, scales, "mxfp8", out)


def mx_pack(codes, gated: bool, fmt="mxfp8", out=None):
    """MX codes [E, rows, K*bits/8] -> the skinny pack layout (gated: W_gateup codes)."""
    bits_, _ = _mx(fmt)
    _need(codes, "codes", torch.uint8)
    if codes.dim() != 3:
        raise ValueError("codes must be [experts, rows, bytes]")
    E, rows, nb = codes.shape
    if out is None:
        out = torch.empty_like(codes)
    _need(out, "out", torch.uint8, tuple(codes.shape), codes.device)
    check("moe_mx_pack", lib().moe_mx_pack(_ptr(codes), E, rows, nb * 8 // bits_, bits_,
                                           int(bool(gated)), _ptr(out), _stream_ptr(codes.device)))
    return out


def mx_tiled_pack(codes, fmt="mxfp8", out=None):
    """MX codes [E, rows, K*bits/8] -> the tiled pack layout (for the tiled,
    prefill kernels; both W_gateup and W_down codes the same way)."""
    bits_, _ = _mx(fmt)
    _need(codes, "codes", torch.uint8)
    if codes.dim() != 3:
        raise ValueError("codes must be [experts, rows, bytes]")
    E, rows, nb = codes.shape
    if out is None:
        out = torch.empty_like(codes)
    _need(out, "out", torch.uint8, tuple(codes.shape), codes.device)
    check("moe_mx_tiled_pack", lib().moe_mx_tiled_pack(_ptr(codes), E, rows, nb * 8 // bits_, bits_,
                                                       _ptr(out), _stream_ptr(codes.device)))
    return out


def gate_up_mx(p: MoeProblem, x_disp, expert_offsets, w_gateup_codes, w_gateup_scales,
               fmt="mxfp8", h=None, packed=False, tiled_packed=False):
    """Gate-up grouped GEMM on MX weights (packed: codes from mx_pack;
    tiled_packed: codes from mx_tiled_pack).  Returns h [cap, I]."""
    bits_, name = _mx(fmt)
    E, H, I = p.num_experts, p.hidden, p.intermediate
    dev = x_disp.device
    cap = _cap(p)
    _need(x_disp, "x_disp", torch.bfloat16, (cap, H))
    _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,), dev)
    _need(w_gateup_codes, "w_gateup_codes", torch.uint8, (E, 2 * I, _mx_code_cols(H, bits_)), dev)
    _need(w_gateup_scales, "w_gateup_scales", torch.uint8, (E, 2 * I, H // 32), dev)
    if h is None:
        h = torch.empty((cap, I), dtype=torch.bfloat16, device=dev)
    _need(h, "h", torch.bfloat16, (cap, I), dev)
    if packed and tiled_packed:
        raise ValueError("packed and tiled_packed are two different layouts")
    if packed or tiled_packed:
        fn = "moe_gate_up_mx_packed" if packed else "moe_gate_up_mx_tiled_packed"
        check(fn, getattr(lib(), fn)(
            ctypes.byref(p), bits_, _ptr(x_disp), _ptr(expert_offsets), _ptr(w_gateup_codes),
            _ptr(w_gateup_scales), _ptr(h), _stream_ptr(dev)))
        return h
    fn = f"moe_gate_up_{name}"
    check(fn, getattr(lib(), fn)(ctypes.byref(p), _ptr(x_disp), _ptr(expert_offsets),
                                 _ptr(w_gateup_codes), _ptr(w_gateup_scales), _ptr(h),
                                 _stream_ptr(dev)))
    return h


def gate_up_mxfp8(p: MoeProblem, x_disp, expert_offsets, w_gateup_codes, w_gateup_scales, h=None):
    return gate_up_mx(p, x_disp, expert_offsets, w_gateup_codes, w_gateup_scales, "mxfp8", h)


def forward_mx(p: MoeProblem, x, topk_ids, topk_weights, w_gateup_codes, w_gateup_scales,
               w_down_codes, w_down_scales, fmt="mxfp8", num_tokens_dev=None,
               expert_offsets=None, out=None, workspace=None, packed=False, tiled_packed=False):
    """The routed-expert layer on MX expert weights (packed: codes from mx_pack;
    tiled_packed: codes from mx_tiled_pack).  Returns (out, expert_offsets)."""
    if packed and tiled_packed:
        raise ValueError("packed and tiled_packed are two different layouts")
    bits_, name = _mx(fmt)
    T, K, E, H, I = p.num_tokens, p.top_k, p.num_experts, p.hidden, p.intermediate
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, H))
    _need(topk_ids, "topk_ids", torch.int32, (T, K), dev)
    _need(topk_weights, "topk_weights", torch.float32, (T, K), dev)
    _need(w_gateup_codes, "w_gateup_codes", torch.uint8, (E, 2 * I, _mx_code_cols(H, bits_)), dev)
    _need(w_gateup_scales, "w_gateup_scales", torch.uint8, (E, 2 * I, H // 32), dev)
    _need(w_down_codes, "w_down_codes", torch.uint8, (E, H, _mx_code_cols(I, bits_)), dev)
    _need(w_down_scales, "w_down_scales", torch.uint8, (E, H, I // 32), dev)
    nt = _ntok(num_tokens_dev, dev)
    if expert_offsets is None:
        expert_offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,), dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (T, H), dev)
    ws = make_workspace(p, dev) if workspace is None else workspace
    args = (_ptr(x), _ptr(topk_ids), _ptr(topk_weights), _ptr(w_gateup_codes),
            _ptr(w_gateup_scales), _ptr(w_down_codes), _ptr(w_down_scales), _ptr(nt),
            _ptr(expert_offsets), _ptr(out), _ptr(ws), ws.numel(), _stream_ptr(dev))
    if packed:
        check("moe_forward_mx_packed", lib().moe_forward_mx_packed(ctypes.byref(p), bits_, *args))
    elif tiled_packed:
        check("moe_forward_mx_tiled_packed",
              lib().moe_forward_mx_tiled_packed(ctypes.byref(p), bits_, *args))
    else:
        fn = f"moe_forward_{name}"
        check(fn, getattr(lib(), fn)(ctypes.byref(p), *args))
    return out, expert_offsets


def forward_mxfp8(p: MoeProblem, x, topk_ids, topk_weights, w_gateup_codes, w_gateup_scales,
                  w_down_codes, w_down_scales, num_tokens_dev=None, expert_offsets=None, out=None,
                  workspace=None):
    return forward_mx(p, x, topk_ids, topk_weights, w_gateup_codes, w_gateup_scales, w_down_codes,
                      w_down_scales, "mxfp8", num_tokens_dev, expert_offsets, out, workspace)


class MoEGraph:
    """One moe_forward recorded into a HIP graph with fixed buffers; replay with
    launch() after writing new inputs (and *num_tokens_dev) into them."""

    def __init__(self, p: MoeProblem, x, topk_ids, topk_weights, w_gateup, w_down,
                 num_tokens_dev=None, expert_offsets=None, out=None, workspace=None):
        nt, offsets, out, ws = _forward_args(p, x, topk_ids, topk_weights, w_gateup, w_down,
                                             num_tokens_dev, expert_offsets, out, workspace)
        self.p = p
        self.device = x.device
        # keep every buffer alive as long as the graph
        self._keep = (x, topk_ids, topk_weights, w_gateup, w_down, nt, offsets, out, ws)
        self.out, self.expert_offsets, self.workspace = out, offsets, ws
        h = ctypes.c_void_p()
        torch.cuda.synchronize(self.device)
        check("moe_graph_create", lib().moe_graph_create(
            ctypes.byref(p), _ptr(x), _ptr(topk_ids), _ptr(topk_weights), _ptr(w_gateup),
            _ptr(w_down), _ptr(nt), _ptr(offsets), _ptr(out), _ptr(ws), ws.numel(),
            ctypes.byref(h)))
        self._h = h

    def launch(self):
        check("moe_graph_launch", lib().moe_graph_launch(self._h, _stream_ptr(self.device)))
        return self.out

    def close(self):
        if self._h is not None and self._h.value:
            check("moe_graph_destroy", lib().moe_graph_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
