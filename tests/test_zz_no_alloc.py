"""moe_forward_noalloc, whose workspace is the library's own device array,
against moe_forward with a caller workspace (through the C ABI): outputs and
expert_offsets equal bit for bit on consecutive calls of decreasing size
(the array keeps the previous call's contents), covering the tiled plan, the
multi-launch skinny plan and the fused tiny path, with a device token count;
output rows past T_v stay untouched; and a problem whose workspace exceeds
the array is refused without writing anything."""
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mixture_experts_routed_02_amd as moe
    from mixture_experts_routed_02_amd import _lib, ops

DEV = "cuda:0"
SENTINEL = 0x7FC1     # a NaN bit pattern no kernel writes


def case(T, K, E, H, I, seed, lo=0, hi=None):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((T, H), generator=g).to(torch.bfloat16)
    wgu = (torch.randn((E, 2 * I, H), generator=g) * H ** -0.5).to(torch.bfloat16)
    wd = (torch.randn((E, H, I), generator=g) * I ** -0.5).to(torch.bfloat16)
    ids = torch.randint(lo, E if hi is None else hi, (T, K), generator=g, dtype=torch.int32)
    w = torch.softmax(torch.randn((T, K), generator=g), dim=1)
    return [t.to(DEV) for t in (x, ids, w, wgu, wd)]


def sentinel(T, H):
    o = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    o.view(torch.int16).fill_(SENTINEL)
    return o


def compare(p, x, ids, w, wgu, wd, tv=None):
    T, H, E = p.num_tokens, p.hidden, p.num_experts
    nt = None if tv is None else torch.tensor([tv], dtype=torch.int32, device=DEV)
    ref = sentinel(T, H)
    ref_off = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    ops.forward(p, x, ids, w, wgu, wd, num_tokens_dev=nt, expert_offsets=ref_off, out=ref,
                workspace=ops.make_workspace(p, DEV))
    got = sentinel(T, H)
    got_off = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    ops.forward_noalloc(p, x, ids, w, wgu, wd, num_tokens_dev=nt, expert_offsets=got_off,
                        out=got)
    torch.cuda.synchronize()
    tvv = T if tv is None else tv
    assert torch.equal(got_off, ref_off)
    assert int(got_off[-1]) > 0
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    assert bool((got[tvv:].view(torch.int16) == SENTINEL).all())


def test_noalloc_equals_forward_on_calls_of_decreasing_size():
    # call 1: the static-capacity layer (2048-token buffer, 16384 rows of
    # capacity, 128 experts, top-8, 2048 x 768), T_v = 1531 on the device
    cfg = W.CONFIGS["static_capacity"]
    T, K, E, H, I = cfg.num_tokens, cfg.top_k, cfg.num_experts, cfg.hidden, cfg.intermediate
    p = moe.problem(T, K, E, H, I, cfg.capacity)
    assert moe.workspace_size(p) <= _lib.NOALLOC_MAX_WORKSPACE
    wgu, wd = W.make_weights(cfg, 5, DEV)
    ids, w = W.make_routing(cfg, 5)
    x = W.make_x(cfg, 5)
    print("[noalloc] static capacity T_v=1531", flush=True)
    compare(p, x.to(DEV), ids.to(DEV), w.to(DEV), wgu, wd, tv=1531)
    del wgu, wd
    # call 2, smaller: 300 tokens, top-4 of 16 experts with dropped ids
    # (multi-launch dispatch, skinny plan forced, then the tiled 64 plan)
    for hint in (1, 2):
        print(f"[noalloc] 300 x top-4, hint {hint}", flush=True)
        compare(moe.problem(300, 4, 16, 512, 384, 0, hint), *case(300, 4, 16, 512, 384, 6, -1, 18))
    # call 3, smaller still: one token, top-6 of 96 (the fused tiny path)
    print("[noalloc] 1 x top-6 of 96", flush=True)
    compare(moe.problem(1, 6, 96, 256, 1024), *case(1, 6, 96, 256, 1024, 7, 0, 100))


def test_noalloc_refuses_oversize_and_writes_nothing():
    p = moe.problem(4096, 2, 8, 4096, 14336)
    assert moe.workspace_size(p) > _lib.NOALLOC_MAX_WORKSPACE
    x = torch.zeros((4096, 4096), dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros((4096, 2), dtype=torch.int32, device=DEV)
    w = torch.zeros((4096, 2), dtype=torch.float32, device=DEV)
    wgu = torch.zeros((8, 2 * 14336, 4096), dtype=torch.bfloat16, device=DEV)
    wd = torch.zeros((8, 4096, 14336), dtype=torch.bfloat16, device=DEV)
    out = sentinel(4096, 4096)
    off = torch.full((9,), -7, dtype=torch.int32, device=DEV)
    with pytest.raises(moe.MoeError) as err:
        ops.forward_noalloc(p, x, ids, w, wgu, wd, expert_offsets=off, out=out)
    assert err.value.status == _lib.MOE_ERROR_NOT_SUPPORTED
    torch.cuda.synchronize()
    assert bool((out.view(torch.int16) == SENTINEL).all())
    assert bool((off == -7).all())
