"""Parity of the MX-weight paths (MXFP8 and MXFP4, through the C ABI) with the
CPU oracle.

* quantization: codes and scales bit for bit against oracle.mxfp8_quantize /
  oracle.mxfp4_quantize, with planted rounding ties, saturating values, zeros,
  -0 and tiny blocks;
* dequantization: every code byte under a range of scales, bit for bit
  against the oracle's decoding (the conversion the expert kernels use);
* the layer: moe_forward_mxfp8 / moe_forward_mxfp4 against the oracle's layer
  on the same codes (to the floating-point bar of helpers.check_close), on
  small ragged shapes through every path (fused dispatch + tiny down/combine,
  fused dispatch + skinny down, multi-launch dispatch), the expert-parallel
  decode share at full size (sampled tokens), a device token count and
  dropped ids.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import bits, check_close, f64, sample_tokens

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mixture_experts_routed_02_amd as moe
    from mixture_experts_routed_02_amd import ops

DEV = "cuda:0"
FMTS = ["mxfp8", "mxfp4"]
ORACLE = {
    "mxfp8": (oracle.mxfp8_quantize, oracle.mxfp8_to_f64, oracle.forward_mxfp8,
              oracle.forward_tokens_mxfp8),
    "mxfp4": (oracle.mxfp4_quantize, oracle.mxfp4_to_f64, oracle.forward_mxfp4,
              oracle.forward_tokens_mxfp4),
}


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def u8(t):
    return t.detach().cpu().contiguous().numpy()


def rand_bf16(shape, std, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(torch.bfloat16)


# ---------------------------------------------------------------------------
# quantize / dequantize
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape,std,seed", [((64, 256), 1.0, 0), ((3, 5, 7168), 7168 ** -0.5, 1),
                                            ((128, 96), 300.0, 2), ((7, 32), 1e-38, 3)])
def test_quantize_bitexact(fmt, shape, std, seed):
    w = rand_bf16(shape, std, seed).to(torch.float32)
    flat = w.view(-1)
    if flat.numel() >= 64:
        flat[:8] = torch.tensor([272.0, 464.0, 496.0, -480.0, 1.0, 1.0625, -0.0, 0.0])
        flat[64:72] = torch.tensor([2.5, 5.0, 0.25, 1.25, 7.0, -6.5, -0.0, 3.5])
        flat[32:64] = 0.0                    # an all-zero block
        flat[40] = -0.0
    w = w.to(torch.bfloat16)
    codes, scales = ops.mx_quantize(w.to(DEV), fmt)
    ref_c, ref_s = ORACLE[fmt][0](bits(w))
    assert np.array_equal(u8(scales), ref_s)
    assert np.array_equal(u8(codes), ref_c)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("scale", [10, 60, 100, 120, 127, 128, 200, 246])
def test_dequantize_every_code(fmt, scale):
    codes = np.tile(np.arange(256, dtype=np.uint8), 4).reshape(8, 128)   # every byte value
    K = 128 if fmt == "mxfp8" else 256
    scales = np.full((8, K // 32), scale, dtype=np.uint8)
    got = ops.mx_dequantize(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV), fmt)
    got = bits(got)
    ref = ORACLE[fmt][1](codes, scales)
    nan = np.isnan(ref)
    assert np.all(np.isnan(oracle.bf16_to_f64(got[nan])))
    assert np.array_equal(got[~nan], oracle.f64_to_bf16_bits(ref[~nan]))


# ---------------------------------------------------------------------------
# the layer
# ---------------------------------------------------------------------------
def quantized_case(fmt, T, K, E, H, I, seed, lo=0, hi=None):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((T, H), generator=g).to(torch.bfloat16)
    wgu = (torch.randn((E, 2 * I, H), generator=g) * H ** -0.5).to(torch.bfloat16)
    wd = (torch.randn((E, H, I), generator=g) * I ** -0.5).to(torch.bfloat16)
    ids = torch.randint(lo, E if hi is None else hi, (T, K), generator=g, dtype=torch.int32)
    w = torch.softmax(torch.randn((T, K), generator=g), dim=1)
    qgu, sgu = ORACLE[fmt][0](bits(wgu))
    qd, sd = ORACLE[fmt][0](bits(wd))
    return x, ids, w, qgu, sgu, qd, sd


def run_forward(fmt, p, x, ids, w, qgu, sgu, qd, sd, nt=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    out, off = ops.forward_mx(p, x.to(DEV), ids.to(DEV), w.to(DEV), t(qgu), t(sgu), t(qd), t(sd),
                              fmt, num_tokens_dev=nt)
    return out, off


SMALL = {
    # name: (T, K, E, H, I, id_lo, id_hi) -- which launches the forward takes
    "fused_tiny_down": (1, 6, 12, 256, 1024, 0, 48),      # T*K <= 8, I % 1024 == 0
    "fused_skinny_down": (64, 2, 8, 256, 512, 0, 8),      # T*K <= 1024
    "fused_ragged": (97, 3, 5, 384, 640, -1, 6),
    "multi_launch": (300, 4, 16, 512, 384, -1, 18),       # T*K > 1024
    "many_experts": (40, 2, 128, 256, 256, 0, 128),
}


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name", list(SMALL))
def test_forward_mx_small(fmt, name):
    T, K, E, H, I, lo, hi = SMALL[name]
    x, ids, w, qgu, sgu, qd, sd = quantized_case(fmt, T, K, E, H, I, 11, lo, hi)
    p = moe.problem(T, K, E, H, I)
    out, off = run_forward(fmt, p, x, ids, w, qgu, sgu, qd, sd)
    _, ref_off, _, _ = oracle.dispatch(ids.numpy(), E)
    assert np.array_equal(off.cpu().numpy(), ref_off)
    ref = ORACLE[fmt][2](bits(x), ids.numpy(), w.numpy(), qgu, sgu, qd, sd)
    check_close(f64(out), ref, name)
    # the same call again gives the same bits (no state carried between calls)
    out2, _ = run_forward(fmt, p, x, ids, w, qgu, sgu, qd, sd)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("fmt", FMTS)
def test_forward_mx_device_token_count_and_dropped(fmt):
    T, K, E, H, I = 200, 4, 16, 256, 256
    x, ids, w, qgu, sgu, qd, sd = quantized_case(fmt, T, K, E, H, I, 12, -2, 20)
    p = moe.problem(T, K, E, H, I)
    for tv in (0, 1, 77, 200):
        nt = torch.tensor([tv], dtype=torch.int32, device=DEV)
        out, off = run_forward(fmt, p, x, ids, w, qgu, sgu, qd, sd, nt)
        _, ref_off, _, _ = oracle.dispatch(ids.numpy(), E, tv)
        assert np.array_equal(off.cpu().numpy(), ref_off)
        ref = ORACLE[fmt][2](bits(x), ids.numpy(), w.numpy(), qgu, sgu, qd, sd, tv)
        check_close(f64(out[:tv]), ref[:tv], f"tv={tv}")
    # a token with no local expert gets an exact zero row
    ids0 = torch.full((1, 6), 40, dtype=torch.int32)
    x1, _, w1, qgu1, sgu1, qd1, sd1 = quantized_case(fmt, 1, 6, 12, 256, 1024, 13)
    out, off = run_forward(fmt, moe.problem(1, 6, 12, 256, 1024), x1, ids0, w1, qgu1, sgu1, qd1,
                           sd1)
    assert int(off[-1]) == 0 and bool((out == 0).all())


@pytest.mark.parametrize("fmt", FMTS)
def test_gate_up_mx_staged(fmt):
    T, K, E, H, I = 50, 2, 6, 256, 384
    x, ids, w, qgu, sgu, qd, sd = quantized_case(fmt, T, K, E, H, I, 14)
    p = moe.problem(T, K, E, H, I)
    x_disp, off, rs, _ = ops.dispatch(p, x.to(DEV), ids.to(DEV))
    h = ops.gate_up_mx(p, x_disp, off, torch.from_numpy(qgu).to(DEV), torch.from_numpy(sgu).to(DEV),
                       fmt)
    o = off.cpu().numpy()
    R = int(o[-1])
    xr = oracle.bf16_to_f64(bits(x_disp)[:R])
    ref = np.zeros((R, I))
    for e in range(E):
        a, b = int(o[e]), int(o[e + 1])
        if a == b:
            continue
        wgu = ORACLE[fmt][1](qgu[e], sgu[e])
        ref[a:b] = oracle.silu(xr[a:b] @ wgu[:I].T) * (xr[a:b] @ wgu[I:].T)
    check_close(f64(h)[:R], ref, "h")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name,seed", [("ep_decode_T1", 0), ("ep_decode_T8", 1),
                                       ("ep_decode_T32", 2), ("ep_decode_T128", 0)])
def test_forward_mx_ep_decode_full_size(fmt, name, seed):
    """The 96-of-384-expert share at full size: weights drawn and quantized on
    the device; the device quantization of one touched expert's down weights
    is checked bit for bit against the oracle, then the layer on sampled
    tokens."""
    cfg = W.CONFIGS[name]
    T, K, E, H, I = cfg.num_tokens, cfg.top_k, cfg.num_experts, cfg.hidden, cfg.intermediate
    x = W.make_x(cfg, seed)
    ids, w = W.make_routing(cfg, seed)
    wgu, wd = W.make_weights(cfg, seed, DEV)
    qgu, sgu = ops.mx_quantize(wgu, fmt)
    qd, sd = ops.mx_quantize(wd, fmt)
    del wgu, wd
    p = moe.problem(T, K, E, H, I)
    out, off = ops.forward_mx(p, x.to(DEV), ids.to(DEV), w.to(DEV), qgu, sgu, qd, sd, fmt)
    _, ref_off, _, _ = oracle.dispatch(ids.numpy(), E)
    assert np.array_equal(off.cpu().numpy(), ref_off)
    toks = sample_tokens(T, 8 if T <= 8 else 4, seed)
    touched = sorted({int(e) for e in ids.numpy()[toks].ravel() if 0 <= e < E})

    class Lazy:
        def __init__(self, t):
            self.t, self.c = t, {}

        def __len__(self):
            return self.t.shape[0]

        def __getitem__(self, e):
            if e not in self.c:
                self.c[e] = u8(self.t[e])
            return self.c[e]

    Q = [Lazy(qgu), Lazy(sgu), Lazy(qd), Lazy(sd)]
    # the device quantization of one touched expert, bit for bit
    if touched:
        e = touched[0]
        wgu_e, wd_e = W.make_weights(cfg, seed, DEV)
        c, s = ORACLE[fmt][0](bits(wd_e[e]))
        assert np.array_equal(Q[2][e], c) and np.array_equal(Q[3][e], s)
        del wgu_e, wd_e
    ref = ORACLE[fmt][3](bits(x), ids.numpy(), w.numpy(), *Q, toks)
    check_close(f64(out)[toks], ref, name)


# ---------------------------------------------------------------------------
# the tiled (prefill) plans on MX weights: codes staged through LDS and
# dequantized on the fragment reads, the tile's scales in LDS; chosen where
# the bf16 layer takes a tiled plan and K is a multiple of 512 (<= 7168)
# ---------------------------------------------------------------------------
TILED = {
    # name: (T, K, E, H, I, id_lo, id_hi)
    "ragged_64": (300, 4, 16, 512, 512, -1, 18),        # ~75 rows per expert: 64-row tiles
    "gate_only_tiled": (97, 3, 5, 1024, 1536, 0, 5),    # down K = 1536: 512-multiple too
    "large_ragged": (2016, 2, 4, 512, 1024, 0, 4),      # ~1008 rows per expert: 192 x 256
    "many_experts_split": (2048, 2, 64, 512, 512, 0, 64),
}


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name", list(TILED))
@pytest.mark.parametrize("hint", [0, 2, 3, 4])
def test_forward_mx_tiled(fmt, name, hint):
    T, K, E, H, I, lo, hi = TILED[name]
    x, ids, w, qgu, sgu, qd, sd = quantized_case(fmt, T, K, E, H, I, 15, lo, hi)
    p = moe.problem(T, K, E, H, I, 0, hint)
    out, off = run_forward(fmt, p, x, ids, w, qgu, sgu, qd, sd)
    _, ref_off, _, _ = oracle.dispatch(ids.numpy(), E)
    assert np.array_equal(off.cpu().numpy(), ref_off)
    ref = ORACLE[fmt][2](bits(x), ids.numpy(), w.numpy(), qgu, sgu, qd, sd)
    check_close(f64(out), ref, f"{name}/hint{hint}")
    out2, _ = run_forward(fmt, p, x, ids, w, qgu, sgu, qd, sd)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def test_forward_mxfp8_tiled_gate_up_128_rows():
    """I % 128 != 0: the large plan's gate-up on 256 x 128 tiles (4 x 2 waves)
    with MXFP8 codes; the down GEMM (K = I = 320) stays on the skinny
    kernels."""
    T, K, E, H, I = 2016, 2, 4, 512, 320
    x, ids, w, qgu, sgu, qd, sd = quantized_case("mxfp8", T, K, E, H, I, 16, 0, 4)
    p = moe.problem(T, K, E, H, I, 0, 4)
    out, _ = run_forward("mxfp8", p, x, ids, w, qgu, sgu, qd, sd)
    ref = ORACLE["mxfp8"][2](bits(x), ids.numpy(), w.numpy(), qgu, sgu, qd, sd)
    check_close(f64(out), ref, "gate-up 256 x 128")


@pytest.mark.parametrize("fmt", FMTS)
def test_forward_mx_tiled_device_token_count_and_dropped(fmt):
    T, K, E, H, I = 700, 4, 16, 512, 512
    x, ids, w, qgu, sgu, qd, sd = quantized_case(fmt, T, K, E, H, I, 17, -2, 20)
    p = moe.problem(T, K, E, H, I, 0, 4)
    for tv in (0, 1, 333, 700):
        nt = torch.tensor([tv], dtype=torch.int32, device=DEV)
        out, off = run_forward(fmt, p, x, ids, w, qgu, sgu, qd, sd, nt)
        _, ref_off, _, _ = oracle.dispatch(ids.numpy(), E, tv)
        assert np.array_equal(off.cpu().numpy(), ref_off)
        ref = ORACLE[fmt][2](bits(x), ids.numpy(), w.numpy(), qgu, sgu, qd, sd, tv)
        check_close(f64(out[:tv]), ref[:tv], f"tv={tv}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("hint", [2, 4])
def test_gate_up_mx_tiled_staged(fmt, hint):
    T, K, E, H, I = 600, 2, 6, 1024, 512
    x, ids, w, qgu, sgu, qd, sd = quantized_case(fmt, T, K, E, H, I, 18)
    p = moe.problem(T, K, E, H, I, 0, hint)
    x_disp, off, rs, _ = ops.dispatch(p, x.to(DEV), ids.to(DEV))
    h = ops.gate_up_mx(p, x_disp, off, torch.from_numpy(qgu).to(DEV), torch.from_numpy(sgu).to(DEV),
                       fmt)
    o = off.cpu().numpy()
    R = int(o[-1])
    xr = oracle.bf16_to_f64(bits(x_disp)[:R])
    ref = np.zeros((R, I))
    for e in range(E):
        a, b = int(o[e]), int(o[e + 1])
        if a == b:
            continue
        wgu = ORACLE[fmt][1](qgu[e], sgu[e])
        ref[a:b] = oracle.silu(xr[a:b] @ wgu[:I].T) * (xr[a:b] @ wgu[I:].T)
    check_close(f64(h)[:R], ref, f"h hint {hint}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name,seed", [("ep_prefill_T8192", 0), ("ep_prefill_T2048_zipf", 1)])
def test_forward_mx_ep_prefill_full_size(fmt, name, seed):
    """The 96-expert prefill share at full size on device-quantized weights
    (the quantizer is checked bit for bit above): every token against the
    oracle's MX layer."""
    from helpers import oracle_workers
    cfg = W.CONFIGS[name]
    T, K, E, H, I = cfg.num_tokens, cfg.top_k, cfg.num_experts, cfg.hidden, cfg.intermediate
    x = W.make_x(cfg, seed)
    ids, w = W.make_routing(cfg, seed)
    wgu, wd = W.make_weights(cfg, seed, DEV)
    qgu, sgu = ops.mx_quantize(wgu, fmt)
    qd, sd = ops.mx_quantize(wd, fmt)
    del wgu, wd
    torch.cuda.empty_cache()
    p = moe.problem(T, K, E, H, I)
    out, off = ops.forward_mx(p, x.to(DEV), ids.to(DEV), w.to(DEV), qgu, sgu, qd, sd, fmt)
    torch.cuda.synchronize()
    _, ref_off, _, _ = oracle.dispatch(ids.numpy(), E)
    assert np.array_equal(off.cpu().numpy(), ref_off)
    toks = np.arange(T)                                     # every token
    deq = ORACLE[fmt][1]
    widen = lambda e: (deq(u8(qgu[e]), u8(sgu[e])), deq(u8(qd[e]), u8(sd[e])))
    ref = oracle.forward_tokens_widened(bits(x), ids.numpy(), w.numpy(), E, widen, toks,
                                        workers=oracle_workers())
    check_close(f64(out)[toks], ref, f"{fmt} {name}")


# ---------------------------------------------------------------------------
# MX codes in the tiled pack layout (moe_mx_tiled_pack): the layout against a
# numpy re-layout written from its definition, and the tiled MX layers on
# packed codes bit-identical to the row-major ones with the same plan (and
# within the oracle's bar)
# ---------------------------------------------------------------------------
def expected_mx_tiled_pack(codes, fmt):
    """Per expert, group g of G rows (16 for e4m3, 32 for e2m1) and stage s
    (64 values: RBW = 64 or 32 bytes of a row), piece L = row G*g + L/C (C =
    RBW / 16 chunks), bytes RBW*s + 16c .. +15 with c = (L % C) ^ swz(row % 32)."""
    E, rows, nb = codes.shape
    rbw = 64 if fmt == "mxfp8" else 32
    ch, wrows = rbw // 16, 1024 // rbw
    G, S = rows // wrows, nb // rbw
    L = np.arange(64)
    r = wrows * np.arange(G)[:, None] + (L // ch)[None, :]                 # [G, 64]
    rm = r % 32
    swz = (((rm >> 2) & 1) | ((rm >> 3) & 2)) if fmt == "mxfp8" else ((rm >> 4) & 1)
    c = (L % ch)[None, :] ^ swz                                            # [G, 64]
    byte = rbw * np.arange(S)[None, :, None, None] + 16 * c[:, None, :, None] + np.arange(16)
    return codes[:, r[:, None, :, None], byte].reshape(E, rows, nb)        # [E, G, S, 64, 16]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("E,rows,K", [(3, 64, 512), (2, 96, 1024), (1, 2048, 64), (4, 32, 7168)])
def test_mx_tiled_pack_layout(fmt, E, rows, K):
    g = torch.Generator().manual_seed(E * rows + K)
    nb = K * (8 if fmt == "mxfp8" else 4) // 8
    codes = torch.randint(0, 256, (E, rows, nb), generator=g, dtype=torch.uint8)
    got = ops.mx_tiled_pack(codes.to(DEV), fmt)
    assert np.array_equal(got.cpu().numpy(), expected_mx_tiled_pack(codes.numpy(), fmt))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name", list(TILED))
@pytest.mark.parametrize("hint", [0, 2, 3, 4])
def test_forward_mx_tiled_packed(fmt, name, hint):
    T, K, E, H, I, lo, hi = TILED[name]
    x, ids, w, qgu, sgu, qd, sd = quantized_case(fmt, T, K, E, H, I, 19, lo, hi)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    qgu_d, sgu_d, qd_d, sd_d = t(qgu), t(sgu), t(qd), t(sd)
    pgu, pd = ops.mx_tiled_pack(qgu_d, fmt), ops.mx_tiled_pack(qd_d, fmt)
    p = moe.problem(T, K, E, H, I, 0, hint)
    xd, idd, wdv = x.to(DEV), ids.to(DEV), w.to(DEV)
    got, off = ops.forward_mx(p, xd, idd, wdv, pgu, sgu_d, pd, sd_d, fmt, tiled_packed=True)
    # the same tiled plan on row-major codes (the automatic choice, or the
    # 64-row tiled plan where it would be the skinny one)
    ref_hint = hint if hint else (2 if T * K / E <= 24 else 0)
    pr = moe.problem(T, K, E, H, I, 0, ref_hint)
    ref, ref_off = ops.forward_mx(pr, xd, idd, wdv, qgu_d, sgu_d, qd_d, sd_d, fmt)
    assert torch.equal(off, ref_off)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    x_disp, o2, _, _ = ops.dispatch(p, xd, idd)
    h_ref = ops.gate_up_mx(pr, x_disp, o2, qgu_d, sgu_d, fmt)
    h = ops.gate_up_mx(p, x_disp, o2, pgu, sgu_d, fmt, tiled_packed=True)
    R = int(o2[-1])
    assert torch.equal(h[:R].view(torch.int16), h_ref[:R].view(torch.int16))
    ref_o = ORACLE[fmt][2](bits(x), ids.numpy(), w.numpy(), qgu, sgu, qd, sd)
    check_close(f64(got), ref_o, f"{fmt} tiled packed {name}/hint{hint}")


@pytest.mark.parametrize("fmt", FMTS)
def test_forward_mx_tiled_packed_full_size(fmt):
    """EP prefill at 8192 tokens: packed codes bit-identical to row-major."""
    cfg = W.CONFIGS["ep_prefill_T8192"]
    T, K, E, H, I = cfg.num_tokens, cfg.top_k, cfg.num_experts, cfg.hidden, cfg.intermediate
    x = W.make_x(cfg, 2).to(DEV)
    ids, w = (a.to(DEV) for a in W.make_routing(cfg, 2))
    wgu, wd = W.make_weights(cfg, 2, DEV)
    qgu, sgu = ops.mx_quantize(wgu, fmt)
    qd, sd = ops.mx_quantize(wd, fmt)
    del wgu, wd
    torch.cuda.empty_cache()
    p = moe.problem(T, K, E, H, I)
    ref, _ = ops.forward_mx(p, x, ids, w, qgu, sgu, qd, sd, fmt)
    pgu, pd = ops.mx_tiled_pack(qgu, fmt), ops.mx_tiled_pack(qd, fmt)
    got, _ = ops.forward_mx(p, x, ids, w, pgu, sgu, pd, sd, fmt, tiled_packed=True)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
