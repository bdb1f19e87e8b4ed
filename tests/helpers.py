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
