"""moe_forward_single: the tiny-batch layer in one cooperative launch (dispatch
and gate-up, a grid barrier, down and combine), through the C ABI.

* bit for bit against moe_forward (the two-launch tiny path, whose parity
  with the oracle test_gpu_parity checks) on small shapes, a device token
  count, all-dropped ids, and the 96-of-384 decode share at T = 1 over 32
  routing draws, and against the oracle directly;
* many launches in a row (the barrier's state is reused) with no barrier
  timeout recorded;
* problems outside the tiny regime are refused.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import DeviceExperts, bits, check_close, f64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mixture_experts_routed_02_amd as moe
    from mixture_experts_routed_02_amd import ops

DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()
    assert ops.single_launch_status() == 0   # no barrier wait timed out


def case(T, K, E, H, I, seed, lo=0, hi=None):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((T, H), generator=g).to(torch.bfloat16)
    wgu = (torch.randn((E, 2 * I, H), generator=g) * H ** -0.5).to(torch.bfloat16)
    wd = (torch.randn((E, H, I), generator=g) * I ** -0.5).to(torch.bfloat16)
    ids = torch.randint(lo, E if hi is None else hi, (T, K), generator=g, dtype=torch.int32)
    w = torch.softmax(torch.randn((T, K), generator=g), dim=1)
    return x, ids, w, wgu, wd


def sentinel(T, H):
    o = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    o.view(torch.int16).fill_(0x7FC1)
    return o


@pytest.mark.parametrize("T,K,E,H,I,lo,hi,tv,seed", [
    (1, 6, 96, 256, 1024, 0, 384, None, 0),
    (1, 6, 12, 512, 2048, 0, 12, None, 1),     # six local experts
    (2, 4, 8, 128, 1024, 0, 8, None, 2),       # duplicates likely
    (4, 2, 8, 64, 1024, 0, 8, 3, 3),           # device token count
    (1, 6, 8, 64, 1024, 9, 12, None, 4),       # every id dropped: a zero row
    (8, 1, 4, 1024, 1024, -1, 5, 5, 5),
])
def test_single_equals_forward(T, K, E, H, I, lo, hi, tv, seed):
    x, ids, w, wgu, wd = (t.to(DEV) for t in case(T, K, E, H, I, seed, lo, hi))
    p = moe.problem(T, K, E, H, I)
    nt = None if tv is None else torch.tensor([tv], dtype=torch.int32, device=DEV)
    ref, ref_off = ops.forward(p, x, ids, w, wgu, wd, num_tokens_dev=nt, out=sentinel(T, H))
    ws = ops.make_workspace(p, DEV)
    for call in range(3):
        got, off = ops.forward_single(p, x, ids, w, wgu, wd, num_tokens_dev=nt,
                                      out=sentinel(T, H), workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(off, ref_off), call
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), call
    tvv = T if tv is None else tv
    r = oracle.forward(bits(x), ids.cpu().numpy(), w.cpu().numpy(), bits(wgu), bits(wd),
                       num_valid_tokens=tvv)
    check_close(f64(got)[:tvv], r[:tvv], "single launch")


def test_single_ep_decode_T1_draws():
    """The 96-of-384 share at T = 1 (7168 x 3072): 32 routing draws in a row,
    each bit-identical to moe_forward; the oracle on every draw."""
    cfg = W.CONFIGS["ep_decode_T1"]
    T, K, E, H, I = cfg.num_tokens, cfg.top_k, cfg.num_experts, cfg.hidden, cfg.intermediate
    wgu, wd = W.make_weights(cfg, 0, DEV)
    x_h = W.make_x(cfg, 0)
    x = x_h.to(DEV)
    p = moe.problem(T, K, E, H, I)
    ws = ops.make_workspace(p, DEV)
    outs = []
    for d in range(32):
        ids_h, w_h = W.make_routing(cfg, 1000 + d)
        ids, w = ids_h.to(DEV), w_h.to(DEV)
        ref, ref_off = ops.forward(p, x, ids, w, wgu, wd)
        got, off = ops.forward_single(p, x, ids, w, wgu, wd, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(off, ref_off), d
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), d
        outs.append((ids_h, w_h, got.clone()))
    gu, dd = DeviceExperts(wgu), DeviceExperts(wd)
    for d, (ids_h, w_h, got) in enumerate(outs):
        r = oracle.forward_tokens(bits(x_h), ids_h.numpy(), w_h.numpy(), gu, dd, np.arange(T))
        check_close(f64(got), r, f"draw {d}")


def test_single_many_launches():
    T, K, E, H, I = 1, 6, 16, 256, 1024
    x, ids, w, wgu, wd = (t.to(DEV) for t in case(T, K, E, H, I, 9, 0, 16))
    p = moe.problem(T, K, E, H, I)
    ws = ops.make_workspace(p, DEV)
    ref, _ = ops.forward(p, x, ids, w, wgu, wd)
    out = torch.empty_like(ref)
    for _ in range(200):
        ops.forward_single(p, x, ids, w, wgu, wd, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("T,K,E,H,I,hint", [
    (2, 6, 8, 256, 1024, 0),      # T*K = 12 > 8
    (1, 6, 8, 256, 512, 0),       # I % 1024 != 0
    (1, 2, 8, 256, 1024, 4),      # a tiled plan forced
])
def test_single_refuses_other_problems(T, K, E, H, I, hint):
    x, ids, w, wgu, wd = (t.to(DEV) for t in case(T, K, E, H, I, 10))
    with pytest.raises(moe.MoeError) as err:
        ops.forward_single(moe.problem(T, K, E, H, I, 0, hint), x, ids, w, wgu, wd)
    assert err.value.status == moe._lib.MOE_ERROR_NOT_SUPPORTED
