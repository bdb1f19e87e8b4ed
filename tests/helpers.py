"""Shared test helpers: tolerance checks and host views of device tensors.

The numeric bar for floating-point results (relative Frobenius error <= 1e-2
and max |err| <= 2e-2 * max|ref| over the checked rows) is the one the
routed-expert path is specified against; bf16 h, y and out each add at most
half an ulp (2^-9 relative), so an fp32-accumulated kernel lands near 0.3-0.5%
Frobenius error.  Integer results (dispatch) are compared bit for bit.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

FRO_TOL = 1e-2
MAX_TOL = 2e-2


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return oracle.bf16_to_f64(bits(t))
    return t.detach().to("cpu").double().numpy()


def check_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    """The floating-point bar; an all-zero reference demands an all-zero result."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rmax = np.abs(ref).max() if ref.size else 0.0
    if rmax == 0.0:
        assert np.all(got == 0.0), f"{what}: reference is zero but result is not"
        return 0.0, 0.0
    err = got - ref
    fro = float(np.linalg.norm(err) / np.linalg.norm(ref))
    mx = float(np.abs(err).max() / rmax)
    assert fro <= FRO_TOL and mx <= MAX_TOL, f"{what}: rel_fro={fro:.3e} max_rel={mx:.3e}"
    return fro, mx


class DeviceExperts:
    """Indexable by expert id -> bf16 bits (numpy) of that expert's weight
    slice, copied from the device on first use; len() = number of experts."""

    def __init__(self, w: torch.Tensor):
        self.w = w
        self.cache = {}

    def __len__(self):
        return self.w.shape[0]

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = bits(self.w[e])
        return self.cache[e]


def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    """n distinct token indices spread over [0, T), always including the first
    and last token."""
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, T - 1], mid]))


def covering_tokens(topk_ids, num_experts: int, n: int, seed: int = 0,
                    tile_rows=(64, 128, 192, 256)) -> np.ndarray:
    """At least n distinct tokens (all of them if T <= n) that include, for
    every expert holding rows: the token of its first and of its last
    dispatched row, and the token of the first row of its last m-tile for
    each tile height in tile_rows (the rows where a ragged last tile starts).
    The rest are drawn uniformly; the first and last token are always in."""
    ids = np.asarray(topk_ids)
    T, K = ids.shape
    if T <= n:
        return np.arange(T)
    _, off, rs, _ = oracle.dispatch(ids, num_experts, T)
    want = {0, T - 1}
    for e in range(num_experts):
        m = int(off[e + 1] - off[e])
        if m == 0:
            continue
        rows = {int(off[e]), int(off[e + 1]) - 1}
        rows.update(int(off[e]) + ((m - 1) // bm) * bm for bm in tile_rows)
        want.update(int(rs[r]) // K for r in rows)
    rng = np.random.default_rng(seed)
    rest = np.setdiff1d(np.arange(T), np.fromiter(want, dtype=np.int64))
    extra = max(0, n - len(want))
    if extra:
        want.update(int(t) for t in rng.choice(rest, size=min(extra, rest.size), replace=False))
    return np.array(sorted(want), dtype=np.int64)


def oracle_workers() -> int:
    """Threads for the oracle's per-expert products (the host's cores, at most 16)."""
    import os
    return max(1, min(16, os.cpu_count() or 1))


class WidenedExperts:
    """widen(e) for oracle.forward_tokens_widened: expert e's weights of the
    device tensors w_gateup [E, 2I, H] and w_down [E, H, I], copied to the host
    and widened with oracle.bf16_to_f64 once, then kept for later calls."""

    def __init__(self, w_gateup: torch.Tensor, w_down: torch.Tensor):
        self.wgu, self.wd = w_gateup, w_down
        self.cache = {}

    def __len__(self):
        return self.wgu.shape[0]

    def __call__(self, e):
        e = int(e)
        hit = self.cache.get(e)
        if hit is None:
            hit = (oracle.bf16_to_f64(bits(self.wgu[e])), oracle.bf16_to_f64(bits(self.wd[e])))
            self.cache[e] = hit
        return hit
