"""GPU parity of the router top-k (moe_router_topk) against the float64
oracle: ids bit for bit (the selection compares the same fp32 values on both
sides), weights within a few fp32 ulps, rows past the device-side token count
untouched, and the Mixtral-style workload's own routing reproduced from its
logits."""
import numpy as np
import pytest
import torch

import mixture_experts_routed_02_amd as moe
import oracle
import workloads as W
from mixture_experts_routed_02_amd import ops

from helpers import DeviceExperts, bits, check_close, f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
W_TOL = 2e-6   # fp32 exp/divide against float64: a few ulps of values <= 1


def _logits(T, E, seed, ties):
    g = torch.Generator().manual_seed(seed)
    lg = torch.randn((T, E), generator=g, dtype=torch.float32)
    if ties:                      # many equal values: the index decides
        lg = torch.round(lg * 2)
    return lg


@pytest.mark.parametrize("T,E,K,seed,ties", [
    (4096, 8, 2, 0, False),       # Mixtral-style routing
    (333, 96, 6, 1, False),
    (100, 64, 64, 2, False),      # K = E = one wave's width
    (257, 16, 5, 3, True),
    (64, 512, 64, 4, False),      # largest E and K
    (50, 200, 7, 5, True),        # E not a multiple of 64
    (9, 1, 1, 6, False),
])
def test_router_vs_oracle(T, E, K, seed, ties):
    lg = _logits(T, E, seed, ties)
    p = moe.problem(T, K, E, 64, 64)
    ids, w = ops.router_topk(p, lg.to(DEV))
    oi, ow = oracle.router_topk(lg.numpy(), K)
    assert np.array_equal(ids.cpu().numpy(), oi)
    assert np.abs(w.cpu().numpy().astype(np.float64) - ow).max() <= W_TOL


def test_router_signed_zero_and_device_token_count():
    lg = torch.tensor([[-0.0, 0.0, -1.0, 3.0], [1.0, 1.0, 1.0, 1.0], [2.0, -0.0, 0.0, 2.0]],
                      dtype=torch.float32)
    T, E, K = 3, 4, 3
    p = moe.problem(T, K, E, 64, 64)
    nt = torch.tensor([2], dtype=torch.int32, device=DEV)
    ids = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T, K), float("nan"), dtype=torch.float32, device=DEV)
    ops.router_topk(p, lg.to(DEV), num_tokens_dev=nt, topk_ids=ids, topk_weights=w)
    oi, ow = oracle.router_topk(lg.numpy(), K, num_valid_tokens=2)
    assert ids[:2].cpu().tolist() == oi.tolist() == [[3, 0, 1], [0, 1, 2]]
    assert np.abs(w[:2].cpu().numpy() - ow).max() <= W_TOL
    assert ids[2].cpu().tolist() == [-7, -7, -7]          # row past T_v untouched
    assert torch.isnan(w[2]).all()


def test_router_feeds_the_layer():
    """Router on the Mixtral-style workload's logits: the workload's own ids
    exactly, and the layer fed by the router's outputs agrees with the layer
    fed by the workload's routing (same rows, weights within fp32 rounding)."""
    cfg = W.CONFIGS["tiny"]
    T, K, E, H, I = cfg.num_tokens, cfg.top_k, cfg.num_experts, cfg.hidden, cfg.intermediate
    d = W.make_inputs(cfg, 1)
    lg = W.make_logits(cfg, 1)
    p = moe.problem(T, K, E, H, I)
    ids, w = ops.router_topk(p, lg.to(DEV))
    assert torch.equal(ids.cpu(), d["topk_ids"])
    assert (w.cpu() - d["topk_weights"]).abs().max().item() <= W_TOL
    x, wgu, wd = d["x"].to(DEV), d["w_gateup"].to(DEV), d["w_down"].to(DEV)
    out_r, _ = ops.forward(p, x, ids, w, wgu, wd)
    out_g, _ = ops.forward(p, x, d["topk_ids"].to(DEV), d["topk_weights"].to(DEV), wgu, wd)
    ref = oracle.forward(bits(d["x"]), d["topk_ids"].numpy(), d["topk_weights"].numpy(),
                         bits(d["w_gateup"]), bits(d["w_down"]))
    check_close(f64(out_r), ref, "router-fed layer")
    check_close(f64(out_g), ref, "generator-fed layer")


# ---------------------------------------------------------------------------
# the router fused ahead of dispatch (moe_router_dispatch, moe_forward_logits)
# ---------------------------------------------------------------------------
def _check_fused_dispatch(lg, T, K, E, G, tv=None, ties=False):
    p = moe.problem(T, K, E, 64, 64)
    x = torch.randn((T, 64), generator=torch.Generator().manual_seed(T)).to(torch.bfloat16)
    nt = None if tv is None else torch.tensor([tv], dtype=torch.int32, device=DEV)
    ids = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T, K), float("nan"), dtype=torch.float32, device=DEV)
    ids, w, x_disp, off, rs, tr = ops.router_dispatch(p, lg.to(DEV), x.to(DEV), num_tokens_dev=nt,
                                                      topk_ids=ids, topk_weights=w)
    tvv = T if tv is None else tv
    # ids bit for bit against the oracle's router, weights within fp32 rounding
    oi, ow = oracle.router_topk(lg.numpy(), K, num_valid_tokens=tvv)
    assert np.array_equal(ids[:tvv].cpu().numpy(), oi)
    assert np.abs(w[:tvv].cpu().numpy().astype(np.float64) - ow).max() <= W_TOL
    # and bit for bit against the standalone router kernel
    pr = moe.problem(T, K, G, 64, 64)
    ids_r = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
    w_r = torch.full((T, K), float("nan"), dtype=torch.float32, device=DEV)
    ops.router_topk(pr, lg.to(DEV), num_tokens_dev=nt, topk_ids=ids_r, topk_weights=w_r)
    assert torch.equal(ids[:tvv], ids_r[:tvv])
    assert torch.equal(w[:tvv].view(torch.int32), w_r[:tvv].view(torch.int32))
    assert bool((ids[tvv:] == -7).all()) and bool(torch.isnan(w[tvv:]).all())
    # the dispatch of those ids (global ids >= E dropped), exact
    full = np.full((T, K), -1, dtype=np.int32)
    full[:tvv] = oi
    _, o_off, o_rs, o_tr = oracle.dispatch(full, E, tvv)
    assert np.array_equal(off.cpu().numpy(), o_off)
    R = int(o_off[-1])
    assert np.array_equal(rs[:R].cpu().numpy(), o_rs)
    assert np.array_equal(tr[:tvv * K].cpu().numpy(), o_tr[:tvv * K])
    if R:
        assert torch.equal(x_disp[:R].view(torch.int16).cpu(),
                           x.view(torch.int16)[torch.from_numpy(o_rs // K).long()])


@pytest.mark.parametrize("T,K,E,G,seed,ties,tv", [
    (4096, 2, 8, 8, 0, False, None),       # Mixtral-style: one block, logits in registers
    (4096, 2, 8, 8, 1, True, 3001),        # ties, device token count
    (1, 6, 96, 384, 2, False, None),       # one token, 384 global experts, 96 local
    (1000, 6, 96, 384, 3, False, None),    # one block, logits read from memory
    (3000, 6, 96, 384, 4, False, 2777),    # multi-block: tokens straddle the 4096-assignment chunks
    (20000, 2, 16, 16, 5, True, None),     # multi-block, register path, ties
    (700, 5, 12, 12, 6, False, None),      # K not dividing the chunk, routed counting (ratio 1)
    (1500, 3, 10, 10, 7, False, 1333),     # routed counting over 1024-assignment chunks, K = 3
    (512, 2, 8, 8, 8, False, None),        # T*K = 1024: the single routing block
    (513, 2, 8, 8, 9, True, None),         # one past it
])
def test_router_dispatch_fused(T, K, E, G, seed, ties, tv):
    _check_fused_dispatch(_logits(T, G, seed, ties), T, K, E, G, tv, ties)


@pytest.mark.parametrize("name,hint", [("tiny", 0), ("tiny", 1), ("mixtral", 0)])
def test_forward_logits_equals_router_then_forward(name, hint):
    """moe_forward_logits equals moe_router_topk + moe_forward bit for bit, and
    the oracle's router + layer within tolerance (the Mixtral layer on 256
    tokens)."""
    cfg = W.CONFIGS[name]
    T, K, E, H, I = cfg.num_tokens, cfg.top_k, cfg.num_experts, cfg.hidden, cfg.intermediate
    lg = W.make_logits(cfg, 2)
    x = W.make_x(cfg, 2)
    wgu, wd = W.make_weights(cfg, 2, DEV)
    p = moe.problem(T, K, E, H, I, 0, hint)
    out, off, ids, w = ops.forward_logits(p, lg.to(DEV), x.to(DEV), wgu, wd)
    ids_r, w_r = ops.router_topk(p, lg.to(DEV))
    out_r, off_r = ops.forward(p, x.to(DEV), ids_r, w_r, wgu, wd)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids_r) and torch.equal(w.view(torch.int32), w_r.view(torch.int32))
    assert torch.equal(off, off_r)
    assert torch.equal(out.view(torch.int16), out_r.view(torch.int16))
    oi, ow = oracle.router_topk(lg.numpy(), K)
    toks = np.arange(min(T, 256))
    ref = oracle.forward_tokens(bits(x), oi, ow.astype(np.float32), DeviceExperts(wgu),
                                DeviceExperts(wd), toks)
    check_close(f64(out)[toks], ref, f"{name} from logits")


@pytest.mark.parametrize("T,K,E,G,H,I,tv", [
    (1, 6, 96, 384, 256, 1024, None),      # tiny path: down GEMM with the combine inside
    (5, 6, 96, 384, 256, 1024, 3),         # device token count
    (300, 4, 16, 20, 512, 384, None),      # skinny multi-launch, some ids non-local
])
def test_forward_logits_small_batches(T, K, E, G, H, I, tv):
    g = torch.Generator().manual_seed(T * 7 + G)
    lg = torch.randn((T, G), generator=g)
    x = torch.randn((T, H), generator=g).to(torch.bfloat16)
    wgu = (torch.randn((E, 2 * I, H), generator=g) * H ** -0.5).to(torch.bfloat16)
    wd = (torch.randn((E, H, I), generator=g) * I ** -0.5).to(torch.bfloat16)
    p = moe.problem(T, K, E, H, I)
    nt = None if tv is None else torch.tensor([tv], dtype=torch.int32, device=DEV)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(0x7FC1)
    out, off, ids, w = ops.forward_logits(p, lg.to(DEV), x.to(DEV), wgu.to(DEV), wd.to(DEV),
                                          num_tokens_dev=nt, out=out)
    tvv = T if tv is None else tv
    pr = moe.problem(T, K, G, H, I)
    ids_r, w_r = ops.router_topk(pr, lg.to(DEV), num_tokens_dev=nt)
    out_r = torch.empty_like(out)
    out_r.view(torch.int16).fill_(0x7FC1)
    ops.forward(p, x.to(DEV), ids_r, w_r, wgu.to(DEV), wd.to(DEV), num_tokens_dev=nt, out=out_r)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_r.view(torch.int16))
    oi, ow = oracle.router_topk(lg.numpy(), K, num_valid_tokens=tvv)
    ids_full = np.full((T, K), -1, dtype=np.int32)
    ids_full[:tvv] = oi
    w_full = np.zeros((T, K), dtype=np.float32)
    w_full[:tvv] = ow
    ref = oracle.forward(bits(x), ids_full, w_full, bits(wgu), bits(wd), num_valid_tokens=tvv)
    check_close(f64(out)[:tvv], ref[:tvv], "small batch from logits")
