"""The C ABI without a GPU: the library loads, exports what the header
declares, sizes workspaces, and fails closed on bad arguments before it
enqueues anything (every call below is rejected by host validation, so no
HIP call is made)."""
import ctypes
import os
import re

import pytest

import mixture_experts_routed_02_amd as moe
from mixture_experts_routed_02_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "moe_mi355x.h")

A16 = 0x100000        # fake, 16-byte aligned "device" addresses: never dereferenced
A4 = 0x200004


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) == 37, names
    L = moe.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.EXPORTS)


def test_status_strings():
    for s in (0, 1, 2, 3):
        assert moe.status_string(s).startswith("MOE_")


def test_workspace_sizes():
    p = moe.problem(4096, 2, 8, 4096, 14336)
    n = moe.workspace_size(p)
    cap = 4096 * 2
    assert n >= cap * (14336 + 4096) * 2 + cap * 4 + 4096 * 2 * 4
    assert n % 256 == 0
    big = moe.workspace_size(moe.problem(4096, 2, 8, 4096, 14336, capacity=2 * cap))
    assert big > n
    assert moe.workspace_size(moe.problem(0, 2, 8, 256, 512)) >= 0


@pytest.mark.parametrize("kw,status", [
    (dict(num_tokens=-1), _lib.MOE_ERROR_INVALID_VALUE),
    (dict(top_k=0), _lib.MOE_ERROR_INVALID_VALUE),
    (dict(top_k=65), _lib.MOE_ERROR_NOT_SUPPORTED),
    (dict(num_experts=0), _lib.MOE_ERROR_INVALID_VALUE),
    (dict(num_experts=513), _lib.MOE_ERROR_NOT_SUPPORTED),
    (dict(hidden=250), _lib.MOE_ERROR_NOT_SUPPORTED),
    (dict(intermediate=100), _lib.MOE_ERROR_NOT_SUPPORTED),
    (dict(capacity=127), _lib.MOE_ERROR_INVALID_VALUE),
    (dict(kernel_hint=7), _lib.MOE_ERROR_INVALID_VALUE),
])
def test_bad_problem_rejected(kw, status):
    base = dict(num_tokens=64, top_k=2, num_experts=8, hidden=256, intermediate=512)
    base.update(kw)
    p = moe.problem(**base)
    n = ctypes.c_size_t(0)
    assert moe.lib().moe_workspace_size(ctypes.byref(p), ctypes.byref(n)) == status
    r = moe.lib().moe_forward(ctypes.byref(p), A16, A4, A4, A16, A16, None, A4, A16, A16,
                              1 << 40, None)
    assert r == status


def test_bad_pointers_rejected():
    p = moe.problem(64, 2, 8, 256, 512)
    ws = moe.workspace_size(p)
    L = moe.lib()
    fwd = lambda *a: L.moe_forward(ctypes.byref(p), *a)
    good = [A16, A4, A4, A16, A16, None, A4, A16, A16, ws, None]
    for i in (0, 1, 2, 3, 4, 6, 7, 8):      # each required pointer nulled
        args = list(good)
        args[i] = None
        assert fwd(*args) == _lib.MOE_ERROR_INVALID_VALUE, i
    for i in (0, 3, 4, 7, 8):               # bf16 / workspace pointers misaligned
        args = list(good)
        args[i] = A16 + 2
        assert fwd(*args) == _lib.MOE_ERROR_INVALID_VALUE, i
    args = list(good)
    args[9] = ws - 1                        # workspace too small
    assert fwd(*args) == _lib.MOE_ERROR_INVALID_VALUE
    args = list(good)
    args[5] = A4 + 1                        # misaligned num_tokens_dev
    assert fwd(*args) == _lib.MOE_ERROR_INVALID_VALUE
    # the staged entry points too
    assert L.moe_dispatch(ctypes.byref(p), A16, None, None, A16, A4, A4, A4, A16, ws, None) == 1
    assert L.moe_expert_compute(ctypes.byref(p), A16, A4, A16, A16, A16, A16, ws - 256, None) == 1
    assert L.moe_combine(ctypes.byref(p), A16, A4, A4, None, A16 + 8, None) == 1
    # router: K > E, null and misaligned pointers, all before any launch
    pk = moe.problem(64, 9, 8, 256, 512)
    assert L.moe_router_topk(ctypes.byref(pk), A4, None, A4, A4, None) == 1
    assert L.moe_router_topk(ctypes.byref(p), None, None, A4, A4, None) == 1
    assert L.moe_router_topk(ctypes.byref(p), A4, None, None, A4, None) == 1
    assert L.moe_router_topk(ctypes.byref(p), A4, None, A4, A4 + 1, None) == 1
    assert L.moe_router_topk(ctypes.byref(p), A4, A4 + 2, A4, A4, None) == 1
    assert L.moe_router_topk(ctypes.byref(moe.problem(0, 2, 8, 256, 512)), None, None, None, None,
                             None) == 0   # T = 0: nothing to do
    assert L.moe_graph_launch(None, None) == 1
    assert L.moe_graph_destroy(None) == 1
    h = ctypes.c_void_p()
    assert L.moe_graph_create(ctypes.byref(p), A16, A4, A4, A16, A16, None, A4, A16, A16, 16,
                              ctypes.byref(h)) == 1
    assert h.value is None


def test_mxfp8_entry_points_fail_closed():
    L = moe.lib()
    p = moe.problem(64, 2, 8, 256, 512)
    ws = moe.workspace_size(p)
    fwd = lambda q, *a: L.moe_forward_mxfp8(ctypes.byref(q), *a)
    good = [A16, A4, A4, A16, A16 + 2, A16, A16 + 2, None, A4, A16, A16, ws, None]
    for i in (0, 1, 2, 3, 4, 5, 6, 8, 9, 10):   # each required pointer nulled
        args = list(good)
        args[i] = None
        assert fwd(p, *args) == _lib.MOE_ERROR_INVALID_VALUE, i
    for i, bad in ((3, A16 + 1), (5, A16 + 8), (4, A16 + 1), (6, A16 + 3), (0, A16 + 2)):
        args = list(good)                       # codes 16-B, scales 2-B, x 16-B aligned
        args[i] = bad
        assert fwd(p, *args) == _lib.MOE_ERROR_INVALID_VALUE, i
    args = list(good)
    args[11] = ws - 1
    assert fwd(p, *args) == _lib.MOE_ERROR_INVALID_VALUE
    for hint in (2, 3, 4):                      # codes in the skinny pack layout: skinny plan only
        q = moe.problem(64, 2, 8, 256, 512, kernel_hint=hint)
        assert L.moe_forward_mx_packed(ctypes.byref(q), 8, *good) == _lib.MOE_ERROR_NOT_SUPPORTED
        assert L.moe_gate_up_mx_packed(ctypes.byref(q), 8, A16, A4, A16, A16, A16, None) == 2
    assert L.moe_gate_up_mxfp8(ctypes.byref(p), A16, A4, A16, A16 + 1, A16, None) == 1
    # quantize / dequantize: k a positive multiple of 32, aligned buffers
    assert L.moe_mxfp8_quantize(A16, 4, 48, A16, A16, None) == 1
    assert L.moe_mxfp8_quantize(A16, 4, 0, A16, A16, None) == 1
    assert L.moe_mxfp8_quantize(A16, -1, 32, A16, A16, None) == 1
    assert L.moe_mxfp8_quantize(A16 + 2, 4, 32, A16, A16, None) == 1
    assert L.moe_mxfp8_quantize(A16, 4, 32, A16 + 4, A16, None) == 1
    assert L.moe_mxfp8_quantize(A16, 4, 32, A16, None, None) == 1
    assert L.moe_mxfp8_quantize(None, 0, 32, None, None, None) == 0     # nothing to do
    assert L.moe_mxfp8_quantize(A16, 1 << 36, 1 << 12, A16, A16, None) == 2
    assert L.moe_mxfp8_dequantize(A16 + 1, A16, 4, 32, A16, None) == 1
    assert L.moe_mxfp8_dequantize(A16, A16, 4, 32, A16 + 2, None) == 1
    assert L.moe_mxfp8_dequantize(A16, A16, 4, 33, A16, None) == 1


def test_mxfp4_entry_points_fail_closed():
    L = moe.lib()
    p = moe.problem(64, 2, 8, 256, 512)
    ws = moe.workspace_size(p)
    good = [A16, A4, A4, A16, A16 + 4, A16, A16 + 4, None, A4, A16, A16, ws, None]
    assert L.moe_forward_mxfp4(ctypes.byref(moe.problem(64, 2, 8, 192, 512)), *good) == 2
    assert L.moe_forward_mxfp4(ctypes.byref(moe.problem(64, 2, 8, 256, 320)), *good) == 2
    for i, bad in ((4, A16 + 2), (6, A16 + 2), (3, A16 + 8)):   # scales 4-B, codes 16-B aligned
        args = list(good)
        args[i] = bad
        assert L.moe_forward_mxfp4(ctypes.byref(p), *args) == _lib.MOE_ERROR_INVALID_VALUE, i
    assert L.moe_gate_up_mx_packed(ctypes.byref(moe.problem(64, 2, 8, 256, 512, kernel_hint=4)),
                                   4, A16, A4, A16, A16, A16, None) == 2
    assert L.moe_mxfp4_quantize(A16, 4, 48, A16, A16, None) == 1
    assert L.moe_mxfp4_dequantize(A16, A16, 4, 32, A16 + 2, None) == 1


def test_skinny_pack_entry_points_fail_closed():
    L = moe.lib()
    assert L.moe_skinny_pack(A16, 2, 24, 64, 0, A16 * 2, None) == 1       # rows % 16
    assert L.moe_skinny_pack(A16, 2, 32, 48, 0, A16 * 2, None) == 1       # k % 32
    assert L.moe_skinny_pack(A16, 2, 32, 64, 2, A16 * 2, None) == 1       # gated is 0 or 1
    assert L.moe_skinny_pack(A16, 2, 32, 64, 1, A16, None) == 1           # in place
    assert L.moe_skinny_pack(A16 + 2, 2, 32, 64, 1, A16 * 2, None) == 1   # misaligned
    assert L.moe_skinny_pack(None, 0, 32, 64, 1, None, None) == 0         # nothing to do
    p = moe.problem(64, 2, 8, 256, 512, kernel_hint=2)
    ws = moe.workspace_size(p)
    assert L.moe_forward_packed(ctypes.byref(p), A16, A4, A4, A16, A16, None, A4, A16, A16, ws,
                                None) == 2
    assert L.moe_gate_up_packed(ctypes.byref(p), A16, A4, A16, A16, None) == 2


def test_mx_pack_entry_points_fail_closed():
    L = moe.lib()
    assert L.moe_mx_pack(A16, 2, 32, 64, 6, 0, A16 * 2, None) == 1        # bits 8 or 4
    assert L.moe_mx_pack(A16, 2, 32, 64, 4, 0, A16 * 2, None) == 1        # MXFP4: k % 128
    assert L.moe_mx_pack(A16, 2, 24, 64, 8, 0, A16 * 2, None) == 1        # rows % 16
    assert L.moe_mx_pack(None, 0, 32, 128, 4, 1, None, None) == 0         # nothing to do
    p = moe.problem(64, 2, 8, 256, 512)
    ws = moe.workspace_size(p)
    assert L.moe_forward_mx_packed(ctypes.byref(p), 5, A16, A4, A4, A16, A16, A16, A16, None, A4,
                                   A16, A16, ws, None) == 1
    assert L.moe_gate_up_mx_packed(ctypes.byref(p), 16, A16, A4, A16, A16, A16, None) == 1


def test_mx_tiled_pack_entry_points_fail_closed():
    L = moe.lib()
    assert L.moe_mx_tiled_pack(A16, 2, 32, 64, 6, A16 * 2, None) == 1        # bits 8 or 4
    assert L.moe_mx_tiled_pack(A16, 2, 16, 64, 8, A16 * 2, None) == 1        # rows % 32
    assert L.moe_mx_tiled_pack(A16, 2, 32, 96, 4, A16 * 2, None) == 1        # k % 64
    assert L.moe_mx_tiled_pack(A16, 2, 32, 128, 8, A16 + 64, None) == 1      # overlap
    assert L.moe_mx_tiled_pack(A16 + 8, 2, 32, 128, 8, A16 * 2, None) == 1   # misaligned
    assert L.moe_mx_tiled_pack(None, 0, 32, 128, 4, None, None) == 0         # nothing to do
    # a skinny plan is refused; K outside the tiled MX range (H % 512) too
    p1 = moe.problem(64, 2, 8, 512, 512, kernel_hint=1)
    ws = moe.workspace_size(p1)
    args = (A16, A4, A4, A16, A16, A16, A16, None, A4, A16, A16, ws, None)
    assert L.moe_forward_mx_tiled_packed(ctypes.byref(p1), 8, *args) == 2
    p2 = moe.problem(64, 2, 8, 256, 512, kernel_hint=4)
    assert L.moe_forward_mx_tiled_packed(ctypes.byref(p2), 8, *args) == 2
    assert L.moe_gate_up_mx_tiled_packed(ctypes.byref(p2), 8, A16, A4, A16, A16, A16, None) == 2
    p3 = moe.problem(64, 2, 8, 512, 512, kernel_hint=4)
    assert L.moe_forward_mx_tiled_packed(ctypes.byref(p3), 5, *args) == 1      # bits
    assert L.moe_gate_up_mx_tiled_packed(ctypes.byref(p3), 8, A16, A4, A16, A16 + 1, A16,
                                         None) == 1                         # scales misaligned


def test_skinny_pack_rejects_overlap():
    L = moe.lib()
    n = 2 * 32 * 64 * 2                                                   # bytes of w
    assert L.moe_skinny_pack(A16, 2, 32, 64, 0, A16 + n - 16, None) == 1  # tail overlaps
    assert L.moe_skinny_pack(A16 + 64, 2, 32, 64, 0, A16, None) == 1      # head overlaps
    assert L.moe_mx_pack(A16, 2, 32, 128, 8, 0, A16 + 64, None) == 1


def test_noalloc_refuses_large_workspace_before_touching_the_gpu():
    """moe_forward_noalloc checks the workspace bound on the host first: a
    problem whose moe_forward workspace exceeds the library's array is
    refused with MOE_ERROR_NOT_SUPPORTED (no HIP call is made), and bad
    arguments fail closed as in moe_forward."""
    L = moe.lib()
    big = moe.problem(4096, 2, 8, 4096, 14336)
    assert moe.workspace_size(big) > _lib.NOALLOC_MAX_WORKSPACE
    r = L.moe_forward_noalloc(ctypes.byref(big), A16, A4, A4, A16, A16, None, A4, A16, None)
    assert r == _lib.MOE_ERROR_NOT_SUPPORTED
    fits = moe.problem(2048, 8, 128, 2048, 768, capacity=16384)
    assert moe.workspace_size(fits) <= _lib.NOALLOC_MAX_WORKSPACE
    good = [A16, A4, A4, A16, A16, None, A4, A16, None]
    for i in (0, 1, 2, 3, 4, 6, 7):      # each required pointer nulled
        args = list(good)
        args[i] = None
        assert L.moe_forward_noalloc(ctypes.byref(fits), *args) == _lib.MOE_ERROR_INVALID_VALUE, i
    args = list(good)
    args[0] = A16 + 2                      # misaligned bf16 pointer
    assert L.moe_forward_noalloc(ctypes.byref(fits), *args) == _lib.MOE_ERROR_INVALID_VALUE
    bad = moe.problem(64, 0, 8, 256, 512)
    assert L.moe_forward_noalloc(ctypes.byref(bad), *good) == _lib.MOE_ERROR_INVALID_VALUE
