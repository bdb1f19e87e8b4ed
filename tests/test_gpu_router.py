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

from helpers import bits, check_close, f64

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
