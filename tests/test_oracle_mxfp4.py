"""Pins of the oracle's MXFP4 weight functions (no GPU).

torch has an e2m1 dtype but no conversions for it, so the decoding is pinned
to the OCP E2M1 value set typed from the format's definition (sign, 2
exponent bits with bias 1, 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6) and to
the torch-pinned e4m3 decoding (every e2m1 value is an e4m3 value with the
same sign); quantization by a brute-force nearest-code search with planted
ties and saturating values, the scale in closed form, the error bounds, the
nibble order of the packing, and the layer against the (pinned) BF16 layer on
the dequantized weights.
"""
import numpy as np
import pytest
import torch

import oracle


def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def rand_bf16(shape, std, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float32) * std).to(torch.bfloat16)


def unpack(packed):
    c = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), np.uint8)
    c[..., 0::2] = packed & 15
    c[..., 1::2] = packed >> 4
    return c


def test_e2m1_decode_table():
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    v = oracle.e2m1_to_f64(np.arange(16, dtype=np.uint8))
    assert v[:8].tolist() == mags
    assert v[8:].tolist() == [-m for m in mags]
    assert np.signbit(v[8]) and not np.signbit(v[0])
    # each e2m1 value is the e4m3 value of the same magnitude and sign
    e4 = oracle.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    for c in range(16):
        hit = np.flatnonzero((e4 == v[c]) & (np.signbit(e4) == np.signbit(v[c])))
        assert hit.size == 1


@pytest.mark.parametrize("seed,std", [(0, 1.0), (1, 7168 ** -0.5), (2, 300.0), (3, 1e-30)])
def test_quantize_scale_closed_form(seed, std):
    w = rand_bf16((48, 256), std, seed)
    packed, scales = oracle.mxfp4_quantize(bits(w))
    assert packed.shape == (48, 128) and scales.shape == (48, 8)
    v = w.to(torch.float64).numpy().reshape(48, 8, 32)
    amax = np.abs(v).max(-1)
    ok = amax > 0
    y = amax / oracle.e8m0_to_f64(scales)
    assert np.all((y[ok] >= 4.0) & (y[ok] < 8.0))      # top binade of e2m1
    q = np.abs(oracle.e2m1_to_f64(unpack(packed))).reshape(48, 8, 32).max(-1)
    assert np.all((q[ok] >= 4.0) & (q[ok] <= 6.0))


def test_quantize_is_nearest_code_brute_force():
    w = rand_bf16((16, 128), 1.0, 5).to(torch.float32)
    # one block with amax 7 -> scale 1: ties 2.5 (2 vs 3 -> 2), 5 (4 vs 6 -> 4),
    # 0.25 (0 vs 0.5 -> 0), 1.25 (1 vs 1.5 -> 1), 7 and -6.5 saturate, -0 keeps its sign
    w[0, :8] = torch.tensor([2.5, 5.0, 0.25, 1.25, 7.0, -6.5, -0.0, 3.5])
    w = w.to(torch.bfloat16)
    packed, scales = oracle.mxfp4_quantize(bits(w))
    codes = unpack(packed)
    v = w.to(torch.float64).numpy()
    y = v / np.repeat(oracle.e8m0_to_f64(scales), 32, axis=-1)
    table = oracle.e2m1_to_f64(np.arange(16, dtype=np.uint8))
    for yi, ci, si in zip(y.ravel(), codes.ravel(), bits(w).ravel() >> 15):
        d = np.abs(table - yi)
        best = np.flatnonzero(d == d.min())
        best = [c for c in best if (c >> 3) == si] or list(best)
        if len(best) > 1:
            best = [c for c in best if c % 2 == 0]
        assert ci == best[0], (yi, ci, best)
    assert scales[0, 0] == 127
    assert oracle.e2m1_to_f64(codes[0, :8]).tolist() == [2.0, 4.0, 0.0, 1.0, 6.0, -6.0, 0.0, 4.0]
    assert codes[0, 6] == 8                                      # -0


def test_packing_nibble_order():
    w = torch.zeros((1, 32), dtype=torch.float32)
    w[0, 0], w[0, 1] = 4.0, 0.5                                  # amax 4 -> scale 1
    packed, scales = oracle.mxfp4_quantize(bits(w.to(torch.bfloat16)))
    assert scales[0, 0] == 127
    assert packed[0, 0] == (0b110 | (0b001 << 4))                # value 0 low, value 1 high


def test_dequantize_error_bounds():
    w = rand_bf16((32, 1024), 7168 ** -0.5, 6)
    packed, scales = oracle.mxfp4_quantize(bits(w))
    v = w.to(torch.float64).numpy()
    d = oracle.mxfp4_to_f64(packed, scales)
    s = np.repeat(oracle.e8m0_to_f64(scales), 32, axis=-1)
    y = np.abs(v) / s
    err = np.abs(d - v) / s
    normal = (y >= 1.0) & (y <= 6.0)
    assert np.all(err[normal] <= y[normal] * 0.25)               # half a spacing: 2^(E-2)
    assert np.all(err[y < 1.0] <= 0.25)
    assert np.all(err[y > 6.0] < 2.0)
    assert np.array_equal(oracle.bf16_to_f64(oracle.f64_to_bf16_bits(d)), d)


def test_mxfp4_forward_equals_bf16_forward_on_dequantized_weights():
    T, K, E, H, I = 24, 3, 5, 64, 96
    g = torch.Generator().manual_seed(7)
    x = bits(rand_bf16((T, H), 1.0, 8))
    wgu = bits(rand_bf16((E, 2 * I, H), H ** -0.5, 9))
    wd = bits(rand_bf16((E, H, I), I ** -0.5, 10))
    ids = torch.randint(-1, E + 1, (T, K), generator=g, dtype=torch.int32).numpy()
    w = torch.rand((T, K), generator=g, dtype=torch.float32).numpy()
    pgu, sgu = oracle.mxfp4_quantize(wgu)
    pd, sd = oracle.mxfp4_quantize(wd)
    assert pgu.shape == (E, 2 * I, H // 2) and sd.shape == (E, H, I // 32)
    got = oracle.forward_mxfp4(x, ids, w, pgu, sgu, pd, sd, num_valid_tokens=20)
    wgu_d = oracle.f64_to_bf16_bits(oracle.mxfp4_to_f64(pgu, sgu))
    wd_d = oracle.f64_to_bf16_bits(oracle.mxfp4_to_f64(pd, sd))
    ref = oracle.forward(x, ids, w, wgu_d, wd_d, num_valid_tokens=20)
    assert np.array_equal(got, ref)
    full = oracle.forward(x, ids, w, wgu, wd, num_valid_tokens=20)
    rel = np.linalg.norm(got - full) / np.linalg.norm(full)
    assert 1e-2 < rel < 0.4
