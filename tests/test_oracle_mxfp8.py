"""Pins of the oracle's MXFP8 weight functions against things other than
themselves (no GPU).

The format (FlashInfer PR #3980, MXFP8 backend and the combine-wire notes:
blocks of 32 e4m3 values sharing one e8m0 scale) is pinned by:

* torch's own float8_e4m3fn decoding of all 256 codes, and closed-form values
  of the OCP E4M3 encoding (448, the smallest subnormal, 1.0, NaN, -0);
* torch's float8_e4m3fn rounding (nearest, ties to even) for every in-range
  element the quantizer rounds;
* a brute-force search over all 256 codes for the nearest value of every
  quantized element, with ties to the even code;
* the scale choice in closed form (each block's largest magnitude lands in
  e4m3's top binade, [256, 448]) and the error bounds that choice implies;
* the layer: the MXFP8 forward equals the (already pinned) BF16 forward on the
  dequantized weights, which are exactly representable in bf16.
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


# ---------------------------------------------------------------------------
# e4m3 / e8m0 decoding
# ---------------------------------------------------------------------------
def test_e4m3_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    assert nan.sum() == 2                       # 0x7F and 0xFF only


def test_e4m3_closed_form_values():
    v = oracle.e4m3_to_f64(np.array([0x7E, 0x01, 0x07, 0x08, 0x38, 0x39, 0x80, 0xB8, 0x00], np.uint8))
    assert v[0] == 448.0                        # 0.1111.110 = 1.75 * 2^8
    assert v[1] == 2.0 ** -9                    # smallest subnormal
    assert v[2] == 7 * 2.0 ** -9                # largest subnormal
    assert v[3] == 2.0 ** -6                    # smallest normal
    assert v[4] == 1.0 and v[5] == 1.125
    assert v[6] == 0.0 and np.signbit(v[6])
    assert v[7] == -1.0 and v[8] == 0.0


def test_e8m0_decode():
    v = oracle.e8m0_to_f64(np.array([127, 128, 0, 254, 255], np.uint8))
    assert v[0] == 1.0 and v[1] == 2.0 and v[2] == 2.0 ** -127 and v[3] == 2.0 ** 127
    assert np.isnan(v[4])


# ---------------------------------------------------------------------------
# quantization
# ---------------------------------------------------------------------------
def _blocks(codes, scales):
    K = codes.shape[-1]
    return codes.reshape(-1, K // 32, 32), scales.reshape(-1, K // 32)


@pytest.mark.parametrize("seed,std", [(0, 1.0), (1, 7168 ** -0.5), (2, 300.0), (3, 1e-30)])
def test_quantize_scale_closed_form(seed, std):
    w = rand_bf16((48, 256), std, seed)
    codes, scales = oracle.mxfp8_quantize(bits(w))
    assert codes.shape == (48, 256) and codes.dtype == np.uint8
    assert scales.shape == (48, 8) and scales.dtype == np.uint8
    v = w.to(torch.float64).numpy().reshape(48, 8, 32)
    amax = np.abs(v).max(-1)
    # the block maximum divided by the scale lies in [256, 512): top binade of e4m3
    y = amax / oracle.e8m0_to_f64(scales)
    ok = amax > 0
    assert np.all((y[ok] >= 256.0) & (y[ok] < 512.0))
    # and its quantized code sits in [256, 448]
    q = np.abs(oracle.e4m3_to_f64(codes)).reshape(48, 8, 32).max(-1)
    assert np.all((q[ok] >= 256.0) & (q[ok] <= 448.0))


def test_quantize_rounding_matches_torch_in_range():
    # elements scaled to [-448, 448] round exactly like torch's float8_e4m3fn cast
    w = rand_bf16((64, 512), 0.05, 4)
    codes, scales = oracle.mxfp8_quantize(bits(w))
    v = w.to(torch.float64).numpy()
    y = v / np.repeat(oracle.e8m0_to_f64(scales), 32, axis=-1)
    inr = np.abs(y) <= 448.0
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert inr.mean() > 0.95
    assert np.array_equal(codes[inr], ref[inr])


def test_quantize_is_nearest_code_brute_force():
    w = rand_bf16((16, 128), 1.0, 5)
    # plant exact ties and saturating values: 1.0 * 2^8 * {1.0625, 1.8125, 1.9375}
    wv = w.to(torch.float32)
    wv[0, :4] = torch.tensor([272.0, 464.0, 496.0, -480.0])      # one block: amax 496 -> scale 1
    wv[1, 32:36] = torch.tensor([1.0, 1.0625, 1.1875, -0.0])     # ties at spacing 1/8 -> even
    wv[1, 36] = 256.0                                            # block amax 256 -> scale 1
    w = wv.to(torch.bfloat16)
    codes, scales = oracle.mxfp8_quantize(bits(w))
    v = w.to(torch.float64).numpy()
    y = v / np.repeat(oracle.e8m0_to_f64(scales), 32, axis=-1)
    table = oracle.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    finite = np.where(np.isnan(table), np.inf, table)
    for yi, ci, si in zip(y.ravel(), codes.ravel(), bits(w).ravel() >> 15):
        d = np.abs(finite - yi)
        best = np.flatnonzero(d == d.min())
        # same sign as the input among equal magnitudes (+0/-0), ties to even code
        best = [c for c in best if (c >> 7) == si] or list(best)
        if len(best) > 1:
            best = [c for c in best if c % 2 == 0]
        assert ci == best[0], (yi, ci, best)
    # the planted values: 272 = 256*1.0625 -> tie between 256 and 288 -> 256 (even)
    assert oracle.e4m3_to_f64(codes[0, :4]).tolist() == [256.0, 448.0, 448.0, -448.0]
    assert oracle.e4m3_to_f64(codes[1, 32:36]).tolist() == [1.0, 1.0, 1.25, 0.0]
    assert codes[1, 35] == 0x80                                   # -0 keeps its sign


def test_dequantize_error_bounds():
    w = rand_bf16((32, 1024), 7168 ** -0.5, 6)
    codes, scales = oracle.mxfp8_quantize(bits(w))
    v = w.to(torch.float64).numpy()
    d = oracle.mxfp8_to_f64(codes, scales)
    s = np.repeat(oracle.e8m0_to_f64(scales), 32, axis=-1)
    y = np.abs(v) / s
    err = np.abs(d - v) / s                                     # in units of the scale
    normal = (y >= 2.0 ** -6) & (y <= 448.0)
    # half a spacing: 2^(E-4) relative to the binade, i.e. <= |y| * 2^-4
    assert np.all(err[normal] <= y[normal] * 2.0 ** -4)
    assert np.all(err[y < 2.0 ** -6] <= 2.0 ** -10)
    assert np.all(err[y > 448.0] < 64.0)
    # the dequantized values are exact bf16 values (needed by the device path)
    assert np.array_equal(oracle.bf16_to_f64(oracle.f64_to_bf16_bits(d)), d)


def test_all_zero_block_and_signed_zero():
    w = torch.zeros((2, 64), dtype=torch.bfloat16)
    w[1, 32:] = -0.0
    codes, scales = oracle.mxfp8_quantize(bits(w))
    assert scales.tolist() == [[0, 0], [0, 0]]
    assert np.all(codes[0] == 0) and np.all(codes[1, :32] == 0) and np.all(codes[1, 32:] == 0x80)


# ---------------------------------------------------------------------------
# the layer on MXFP8 weights
# ---------------------------------------------------------------------------
def test_mxfp8_forward_equals_bf16_forward_on_dequantized_weights():
    T, K, E, H, I = 24, 3, 5, 64, 96
    g = torch.Generator().manual_seed(7)
    x = bits(rand_bf16((T, H), 1.0, 8))
    wgu = bits(rand_bf16((E, 2 * I, H), H ** -0.5, 9))
    wd = bits(rand_bf16((E, H, I), I ** -0.5, 10))
    ids = torch.randint(-1, E + 1, (T, K), generator=g, dtype=torch.int32).numpy()
    w = torch.rand((T, K), generator=g, dtype=torch.float32).numpy()
    qgu, sgu = oracle.mxfp8_quantize(wgu)
    qd, sd = oracle.mxfp8_quantize(wd)
    assert sgu.shape == (E, 2 * I, H // 32) and sd.shape == (E, H, I // 32)
    got = oracle.forward_mxfp8(x, ids, w, qgu, sgu, qd, sd, num_valid_tokens=20)
    wgu_d = oracle.f64_to_bf16_bits(oracle.mxfp8_to_f64(qgu, sgu))
    wd_d = oracle.f64_to_bf16_bits(oracle.mxfp8_to_f64(qd, sd))
    ref = oracle.forward(x, ids, w, wgu_d, wd_d, num_valid_tokens=20)
    assert np.array_equal(got, ref)
    # and it stays near the unquantized layer (e4m3 keeps 3 mantissa bits)
    full = oracle.forward(x, ids, w, wgu, wd, num_valid_tokens=20)
    rel = np.linalg.norm(got - full) / np.linalg.norm(full)
    assert 1e-3 < rel < 0.1
