"""Seeded synthetic inputs for the routed-MoE expert path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no dispatch, no GEMM, no SiLU, no combine).  Both the HIP
path and the CPU oracle consume what it returns.

The workloads follow the shapes and distributions of the pages' benchmarks:

* DeepGEMM PR #394, "Performance": 384 experts, top-6, hidden 7168,
  intermediate 3072, no shared experts, deterministic random routing; one
  rank's expert-parallel share is 96 local experts.
* TileOps PR #1738, "Summary"/"Scope": BF16 tight expert-major batches with a
  static capacity and a device-resident valid-row count, replayed as a graph.
* FlashInfer PR #3980, "Accuracy": random data against a dense ground truth.

Every tensor is drawn from its own ``torch.Generator`` seeded with
``(seed, stream)`` so that one part (for instance the 12.7 GB of expert
weights, which are drawn on the GPU when a device is given) can be produced on
another device without changing the others.  Values drawn on a GPU differ from
values drawn on the CPU for the same seed; each run is self-consistent because
the oracle reads the very tensors the GPU path reads.

Routing conventions (the plainest reading of the pages):

* ``softmax_topk``: router logits ~ N(0,1) fp32 over the E experts, the top-k
  by value (lower expert index wins ties), weights = softmax over the k
  selected logits.
* ``ep_uniform``: each token draws k distinct experts uniformly out of the
  global pool (384); only ids below E (96) are local, the rest are passed
  through unchanged and are dropped by the path.  Weights = softmax over k
  N(0,1) logits, not renormalised over the local subset.
* ``ep_zipf``: as ``ep_uniform`` but expert popularity p(rank r) ~ r^-s,
  s = 1.2, with a per-seed random permutation from rank to expert id; k
  distinct experts per token by Gumbel-top-k over log p (sampling without
  replacement).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

# Stream ids of the independent generators.
_S_X, _S_WGU, _S_WD, _S_ROUTE, _S_TV, _S_AUX = 1, 2, 3, 4, 5, 6


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    num_tokens: int          # T: rows of x / out (buffer rows)
    top_k: int               # K
    num_experts: int         # E: local experts (rows of the weight tensors)
    hidden: int              # H
    intermediate: int        # I
    routing: str             # softmax_topk | ep_uniform | ep_zipf
    global_experts: int = 0  # pool the ids are drawn from (0 => E)
    zipf_s: float = 1.2
    capacity: int = 0        # dispatched-row buffer rows (0 => T*K)

    @property
    def pool(self) -> int:
        return self.global_experts or self.num_experts

    @property
    def cap(self) -> int:
        return self.capacity or self.num_tokens * self.top_k

    def with_tokens(self, t: int) -> "MoEConfig":
        return dataclasses.replace(self, num_tokens=t, name=f"{self.name.split('@')[0]}@T{t}")


def _cfg_table():
    c = {}
    c["tiny"] = MoEConfig("tiny", 64, 2, 8, 256, 512, "softmax_topk")
    c["mixtral"] = MoEConfig("mixtral", 4096, 2, 8, 4096, 14336, "softmax_topk")
    for t in (1, 8, 32, 128):
        c[f"ep_decode_T{t}"] = MoEConfig(f"ep_decode_T{t}", t, 6, 96, 7168, 3072, "ep_uniform", 384)
    for t in (2048, 8192):
        c[f"ep_prefill_T{t}"] = MoEConfig(f"ep_prefill_T{t}", t, 6, 96, 7168, 3072, "ep_uniform", 384)
        c[f"ep_prefill_T{t}_zipf"] = MoEConfig(f"ep_prefill_T{t}_zipf", t, 6, 96, 7168, 3072, "ep_zipf", 384)
    # supplementary point of the same shape with about 256 rows per local
    # expert, where one weight pass allows up to 78.5% of the MFMA peak
    c["ep_prefill_T16384"] = MoEConfig("ep_prefill_T16384", 16384, 6, 96, 7168, 3072, "ep_uniform", 384)
    c["static_capacity"] = MoEConfig("static_capacity", 2048, 8, 128, 2048, 768, "ep_uniform", 128,
                                     capacity=16384)
    return c


CONFIGS = _cfg_table()

# Graph replays of the static-capacity workload: T_v ~ U{1..2048}.
STATIC_REPLAYS = 50


def _gen(seed: int, stream: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + stream * 7_919) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def _normal_bf16(shape, std: float, gen: torch.Generator, device) -> torch.Tensor:
    # fp32 N(0, std^2) rounded to bf16 (round to nearest even).
    return (torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std).to(torch.bfloat16)


def make_x(cfg: MoEConfig, seed: int, device="cpu") -> torch.Tensor:
    """x ~ N(0,1), bf16 [T, H]."""
    return _normal_bf16((cfg.num_tokens, cfg.hidden), 1.0, _gen(seed, _S_X, device), device)


def make_weights(cfg: MoEConfig, seed: int, device="cpu"):
    """W_gateup bf16 [E, 2I, H] (rows [0,I) gate, [I,2I) up) ~ N(0, 1/H);
    W_down bf16 [E, H, I] ~ N(0, 1/I).  Drawn one expert at a time so that the
    fp32 temporaries stay small."""
    E, H, I = cfg.num_experts, cfg.hidden, cfg.intermediate
    wgu = torch.empty((E, 2 * I, H), dtype=torch.bfloat16, device=device)
    wd = torch.empty((E, H, I), dtype=torch.bfloat16, device=device)
    g1, g2 = _gen(seed, _S_WGU, device), _gen(seed, _S_WD, device)
    for e in range(E):
        wgu[e] = _normal_bf16((2 * I, H), 1.0 / math.sqrt(H), g1, device)
        wd[e] = _normal_bf16((H, I), 1.0 / math.sqrt(I), g2, device)
    return wgu, wd


def _softmax_rows(z: torch.Tensor) -> torch.Tensor:
    return torch.softmax(z.to(torch.float32), dim=1)


def make_routing(cfg: MoEConfig, seed: int, num_tokens: Optional[int] = None):
    """Returns (topk_ids int32 [T, K], topk_weights fp32 [T, K]) on the CPU.

    ids may lie outside [0, E) for the expert-parallel workloads (non-local
    experts); the path drops them by value."""
    T = cfg.num_tokens if num_tokens is None else num_tokens
    K, G = cfg.top_k, cfg.pool
    g = _gen(seed, _S_ROUTE)
    if cfg.routing == "softmax_topk":
        logits = torch.randn((T, G), generator=g, dtype=torch.float32)
        # Stable sort on -logits: lower index first among equal values.
        ids = torch.argsort(-logits, dim=1, stable=True)[:, :K]
        sel = torch.gather(logits, 1, ids)
        w = _softmax_rows(sel)
    elif cfg.routing == "ep_uniform":
        # k distinct experts uniformly from the pool: prefix of a random permutation.
        keys = torch.rand((T, G), generator=g, dtype=torch.float32)
        ids = torch.argsort(keys, dim=1, stable=True)[:, :K]
        w = _softmax_rows(torch.randn((T, K), generator=g, dtype=torch.float32))
    elif cfg.routing == "ep_zipf":
        ranks = torch.arange(1, G + 1, dtype=torch.float64)
        p = ranks.pow(-cfg.zipf_s)
        p = p / p.sum()
        perm = torch.randperm(G, generator=g)            # rank r -> expert perm[r]
        logp = torch.empty(G, dtype=torch.float64)
        logp[perm] = torch.log(p)
        u = torch.rand((T, G), generator=g, dtype=torch.float64).clamp_(1e-300, 1.0 - 1e-16)
        gumbel = -torch.log(-torch.log(u))
        ids = torch.argsort(-(logp[None, :] + gumbel), dim=1, stable=True)[:, :K]
        w = _softmax_rows(torch.randn((T, K), generator=g, dtype=torch.float32))
    else:
        raise ValueError(f"unknown routing {cfg.routing!r}")
    return ids.to(torch.int32).contiguous(), w.contiguous()


def make_logits(cfg: MoEConfig, seed: int, num_tokens: Optional[int] = None):
    """Router logits fp32 [T, E] of a softmax_topk workload: the very values
    make_routing draws (same generator stream), so that a router applied to
    them must give make_routing's ids and weights."""
    if cfg.routing != "softmax_topk":
        raise ValueError(f"{cfg.name} has no router logits (routing {cfg.routing!r})")
    T = cfg.num_tokens if num_tokens is None else num_tokens
    g = _gen(seed, _S_ROUTE)
    return torch.randn((T, cfg.pool), generator=g, dtype=torch.float32)


def make_static_token_counts(seed: int, replays: int = STATIC_REPLAYS, max_tokens: int = 2048) -> list:
    """T_v for each graph replay of the static-capacity workload, ~ U{1..max_tokens}."""
    g = _gen(seed, _S_TV)
    return [int(v) for v in torch.randint(1, max_tokens + 1, (replays,), generator=g)]


def make_bf16_rows(rows: int, cols: int, seed: int, stream: int = _S_AUX, device="cpu") -> torch.Tensor:
    """Generic N(0,1) bf16 matrix, e.g. a stand-in expert-output batch for a
    combine-only test."""
    return _normal_bf16((rows, cols), 1.0, _gen(seed, stream, device), device)


def make_inputs(cfg: MoEConfig, seed: int, weight_device="cpu"):
    """All inputs of one forward call: dict of x, topk_ids, topk_weights,
    w_gateup, w_down (x and routing on the CPU, weights on ``weight_device``)."""
    x = make_x(cfg, seed)
    wgu, wd = make_weights(cfg, seed, weight_device)
    ids, w = make_routing(cfg, seed)
    return {"x": x, "topk_ids": ids, "topk_weights": w, "w_gateup": wgu, "w_down": wd}


def bf16_bits(t: torch.Tensor):
    """A bf16 tensor's raw bit pattern as a numpy uint16 array (CPU copy)."""
    import numpy as np
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
