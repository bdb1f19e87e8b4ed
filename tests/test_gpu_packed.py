"""The skinny pack layout of bf16 expert weights (through the C ABI):

* the layout itself, bit for bit, against a numpy re-layout written from its
  definition (16-row groups, [k-steps][64 lanes][8 values], gate/up pairing
  for W_gateup);
* the bitwise A/B gate: moe_forward_packed and moe_gate_up_packed equal
  moe_forward / moe_gate_up with the skinny plan on the row-major weights,
  bit for bit, on every launch path (fused dispatch + tiny down/combine,
  fused dispatch + skinny down, multi-launch dispatch), with a device token
  count, and on the full-size expert-parallel decode share;
* the packed layers directly against the oracle: bf16 packed weights, and MX
  codes quantized on the host by the oracle, then packed on the device.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import DeviceExperts, bits, check_close, f64, oracle_workers

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


def expected_pack(w_bits, gated):
    E, rows, K = w_bits.shape
    G, S = rows // 16, K // 32
    l = np.arange(64)
    li, lg = l % 16, l // 16
    g = np.arange(G)[:, None]
    if gated:
        r = np.where(li[None, :] < 8, 8 * g + li[None, :], rows // 2 + 8 * g + li[None, :] - 8)
    else:
        r = 16 * g + li[None, :]                                   # [G, 64]
    k0 = 32 * np.arange(S)[:, None] + 8 * lg[None, :]              # [S, 64]
    kk = k0[:, :, None] + np.arange(8)                             # [S, 64, 8]
    out = w_bits[:, r[:, None, :, None], kk[None, :, :, :]]        # [E, G, S, 64, 8]
    return out.reshape(E, rows, K)


@pytest.mark.parametrize("E,rows,K,gated", [(3, 64, 256, False), (2, 96, 192, True),
                                            (5, 32, 512, True), (1, 2048, 64, False)])
def test_pack_layout(E, rows, K, gated):
    g = torch.Generator().manual_seed(E * rows + K)
    w = torch.randn((E, rows, K), generator=g).to(torch.bfloat16)
    got = ops.skinny_pack(w.to(DEV), gated)
    assert np.array_equal(bits(got), expected_pack(bits(w), gated))


def case(T, K, E, H, I, seed, lo=0, hi=None):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((T, H), generator=g).to(torch.bfloat16)
    wgu = (torch.randn((E, 2 * I, H), generator=g) * H ** -0.5).to(torch.bfloat16)
    wd = (torch.randn((E, H, I), generator=g) * I ** -0.5).to(torch.bfloat16)
    ids = torch.randint(lo, E if hi is None else hi, (T, K), generator=g, dtype=torch.int32)
    w = torch.softmax(torch.randn((T, K), generator=g), dim=1)
    return [t.to(DEV) for t in (x, ids, w, wgu, wd)]


SHAPES = {
    "tiny_down": (1, 6, 12, 256, 1024, 0, 48),         # T*K <= 8, I % 1024 == 0
    "fused_skinny_down": (64, 2, 8, 256, 512, 0, 8),
    "fused_ragged": (97, 3, 5, 192, 320, -1, 6),
    "multi_launch": (300, 4, 16, 512, 384, -1, 18),     # T*K > 1024
    "small_hidden": (20, 2, 4, 320, 256, 0, 4),
}


@pytest.mark.parametrize("name", list(SHAPES))
def test_forward_packed_bit_identical(name):
    T, K, E, H, I, lo, hi = SHAPES[name]
    x, ids, w, wgu, wd = case(T, K, E, H, I, 21, lo, hi)
    p = moe.problem(T, K, E, H, I, 0, moe.HINT_SKINNY)
    ref, ref_off = ops.forward(p, x, ids, w, wgu, wd)
    pgu, pd = ops.skinny_pack(wgu, True), ops.skinny_pack(wd, False)
    got, off = ops.forward_packed(p, x, ids, w, pgu, pd)
    assert torch.equal(off, ref_off)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    # gate-up alone
    x_disp, o2, _, _ = ops.dispatch(p, x, ids)
    h_ref = ops.gate_up(p, x_disp, o2, wgu)
    h = ops.gate_up_packed(p, x_disp, o2, pgu)
    R = int(o2[-1])
    assert torch.equal(h[:R].view(torch.int16), h_ref[:R].view(torch.int16))


def test_forward_packed_device_token_count():
    T, K, E, H, I = 200, 4, 16, 256, 256
    x, ids, w, wgu, wd = case(T, K, E, H, I, 22, -2, 20)
    p = moe.problem(T, K, E, H, I, 0, moe.HINT_SKINNY)
    pgu, pd = ops.skinny_pack(wgu, True), ops.skinny_pack(wd, False)
    for tv in (0, 1, 77, 200):
        nt = torch.tensor([tv], dtype=torch.int32, device=DEV)
        ref, _ = ops.forward(p, x, ids, w, wgu, wd, num_tokens_dev=nt)
        got, _ = ops.forward_packed(p, x, ids, w, pgu, pd, num_tokens_dev=nt)
        assert torch.equal(got[:tv].view(torch.int16), ref[:tv].view(torch.int16)), tv


@pytest.mark.parametrize("name", ["ep_decode_T1", "ep_decode_T32"])
def test_forward_packed_ep_decode_full_size(name):
    cfg = W.CONFIGS[name]
    T, K, E, H, I = cfg.num_tokens, cfg.top_k, cfg.num_experts, cfg.hidden, cfg.intermediate
    x = W.make_x(cfg, 0).to(DEV)
    ids, w = (t.to(DEV) for t in W.make_routing(cfg, 0))
    wgu, wd = W.make_weights(cfg, 0, DEV)
    p = moe.problem(T, K, E, H, I)
    ref, _ = ops.forward(p, x, ids, w, wgu, wd)
    pgu, pd = ops.skinny_pack(wgu, True), ops.skinny_pack(wd, False)
    got, _ = ops.forward_packed(p, x, ids, w, pgu, pd)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


# ---------------------------------------------------------------------------
# MX codes in the pack layout: bit-identical to the row-major MX path (which
# test_gpu_mx checks against the oracle)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("name", ["tiny_down", "fused_skinny_down", "multi_launch"])
def test_forward_mx_packed_bit_identical(fmt, name):
    """Packed MX weights run the skinny kernels only, so the row-major
    reference is pinned to the skinny plan too (left to itself it takes the
    tiled MX kernels where those apply, whose accumulation order differs)."""
    T, K, E, H, I, lo, hi = SHAPES[name]
    x, ids, w, wgu, wd = case(T, K, E, H, I, 23, lo, hi)
    p = moe.problem(T, K, E, H, I, 0, moe.HINT_SKINNY)
    qgu, sgu = ops.mx_quantize(wgu, fmt)
    qd, sd = ops.mx_quantize(wd, fmt)
    ref, ref_off = ops.forward_mx(p, x, ids, w, qgu, sgu, qd, sd, fmt)
    pgu, pd = ops.mx_pack(qgu, True, fmt), ops.mx_pack(qd, False, fmt)
    # the MX pack is the bf16 pack of the code bytes viewed as 16-bit values
    assert np.array_equal(bits(pgu.view(torch.bfloat16)),
                          expected_pack(bits(qgu.view(torch.bfloat16)), True))
    got, off = ops.forward_mx(p, x, ids, w, pgu, sgu, pd, sd, fmt, packed=True)
    assert torch.equal(off, ref_off)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    x_disp, o2, _, _ = ops.dispatch(p, x, ids)
    h_ref = ops.gate_up_mx(p, x_disp, o2, qgu, sgu, fmt)
    h = ops.gate_up_mx(p, x_disp, o2, pgu, sgu, fmt, packed=True)
    R = int(o2[-1])
    assert torch.equal(h[:R].view(torch.int16), h_ref[:R].view(torch.int16))


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("name", ["ep_decode_T1", "ep_decode_T32"])
def test_forward_mx_packed_ep_decode_full_size(fmt, name):
    cfg = W.CONFIGS[name]
    T, K, E, H, I = cfg.num_tokens, cfg.top_k, cfg.num_experts, cfg.hidden, cfg.intermediate
    x = W.make_x(cfg, 1).to(DEV)
    ids, w = (t.to(DEV) for t in W.make_routing(cfg, 1))
    wgu, wd = W.make_weights(cfg, 1, DEV)
    qgu, sgu = ops.mx_quantize(wgu, fmt)
    qd, sd = ops.mx_quantize(wd, fmt)
    del wgu, wd
    p = moe.problem(T, K, E, H, I)
    ref, _ = ops.forward_mx(p, x, ids, w, qgu, sgu, qd, sd, fmt)
    pgu, pd = ops.mx_pack(qgu, True, fmt), ops.mx_pack(qd, False, fmt)
    got, _ = ops.forward_mx(p, x, ids, w, pgu, sgu, pd, sd, fmt, packed=True)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


# ---------------------------------------------------------------------------
# static capacity + graph replay on the packed and MX entry points: every one
# of them only enqueues kernels (no allocation, memset or host read), so a
# caller can record it into a HIP graph and replay it with a new device token
# count; each replay must equal the eager call with that count, bit for bit
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kind", ["packed", "mxfp8", "mxfp4", "mxfp8_packed", "tiled_packed",
                                  "logits"])
def test_graph_replays_with_device_token_count(kind):
    cfg = W.CONFIGS["static_capacity"]
    T, K, E, H, I = cfg.num_tokens, cfg.top_k, cfg.num_experts, cfg.hidden, cfg.intermediate
    x = W.make_x(cfg, 4).to(DEV)
    ids, w = (t.to(DEV) for t in W.make_routing(cfg, 4))
    wgu, wd = W.make_weights(cfg, 4, DEV)
    p = moe.problem(T, K, E, H, I, cfg.capacity)
    if kind == "packed":
        a, b = ops.skinny_pack(wgu, True), ops.skinny_pack(wd, False)
        run = lambda nt, out, off, ws: ops.forward_packed(p, x, ids, w, a, b, nt, off, out, ws)
    elif kind == "tiled_packed":
        a, b = ops.tiled_pack(wgu), ops.tiled_pack(wd)
        run = lambda nt, out, off, ws: ops.forward_tiled_packed(p, x, ids, w, a, b, nt, off, out,
                                                                ws)
    elif kind == "logits":   # the router fused ahead of the dispatch
        lg = torch.randn((T, E), generator=torch.Generator().manual_seed(4)).to(DEV)
        bufs = {}

        def run(nt, out, off, ws):
            ib, wb = bufs.setdefault(out.data_ptr(), (
                torch.full((T, K), -1, dtype=torch.int32, device=DEV),
                torch.zeros((T, K), dtype=torch.float32, device=DEV)))
            ops.forward_logits(p, lg, x, wgu, wd, nt, ib, wb, off, out, ws)
    else:
        fmt = kind.split("_")[0]
        qgu, sgu = ops.mx_quantize(wgu, fmt)
        qd, sd = ops.mx_quantize(wd, fmt)
        packed = kind.endswith("packed")
        if packed:
            qgu, qd = ops.mx_pack(qgu, True, fmt), ops.mx_pack(qd, False, fmt)
        run = lambda nt, out, off, ws: ops.forward_mx(p, x, ids, w, qgu, sgu, qd, sd, fmt, nt, off,
                                                      out, ws, packed=packed)
    nt = torch.tensor([T], dtype=torch.int32, device=DEV)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    off = torch.empty((E + 1,), dtype=torch.int32, device=DEV)
    ws = ops.make_workspace(p, DEV)
    run(nt, out, off, ws)                                  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(nt, out, off, ws)
    ref_out = torch.empty_like(out)
    ref_off = torch.empty_like(off)
    ref_ws = ops.make_workspace(p, DEV)
    for tv in (2048, 1, 700, 0, 1999, 64):
        nt.fill_(tv)
        out.view(torch.int16).fill_(0x7FC1)                # a NaN pattern no kernel writes
        g.replay()
        torch.cuda.synchronize()
        nt_e = torch.tensor([tv], dtype=torch.int32, device=DEV)
        run(nt_e, ref_out, ref_off, ref_ws)                # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(off, ref_off), tv
        assert torch.equal(out[:tv].view(torch.int16), ref_out[:tv].view(torch.int16)), tv
        assert bool((out[tv:].view(torch.int16) == 0x7FC1).all()), tv   # rows >= T_v untouched


# ---------------------------------------------------------------------------
# the packed layers against the oracle directly
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(SHAPES))
def test_forward_packed_vs_oracle(name):
    T, K, E, H, I, lo, hi = SHAPES[name]
    x, ids, w, wgu, wd = case(T, K, E, H, I, 24, lo, hi)
    p = moe.problem(T, K, E, H, I)
    pgu, pd = ops.skinny_pack(wgu, True), ops.skinny_pack(wd, False)
    got, off = ops.forward_packed(p, x, ids, w, pgu, pd)
    ids_h = ids.cpu().numpy()
    _, o_off, _, _ = oracle.dispatch(ids_h, E, T)
    assert np.array_equal(off.cpu().numpy(), o_off)
    ref = oracle.forward(bits(x), ids_h, w.cpu().numpy(), bits(wgu), bits(wd))
    check_close(f64(got), ref, f"packed {name}")


# MXFP4 takes H and I multiples of 128 only; the shapes outside that are
# MXFP8 cases alone
MX_PACKED_CASES = [(fmt, name) for name in SHAPES for fmt in ("mxfp8", "mxfp4")
                   if fmt == "mxfp8" or (SHAPES[name][3] % 128 == 0 and SHAPES[name][4] % 128 == 0)]


@pytest.mark.parametrize("fmt,name", MX_PACKED_CASES)
def test_forward_mx_packed_vs_oracle(fmt, name):
    """MX codes and scales from the oracle's quantizer (host), packed on the
    device, through moe_forward_mx_packed, against the oracle's MX layer."""
    T, K, E, H, I, lo, hi = SHAPES[name]
    x, ids, w, wgu, wd = case(T, K, E, H, I, 25, lo, hi)
    quant = oracle.mxfp8_quantize if fmt == "mxfp8" else oracle.mxfp4_quantize
    cg, sg = quant(bits(wgu))
    cd, sd = quant(bits(wd))
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    qgu, sgu, qd, sdd = d(cg), d(sg), d(cd), d(sd)
    p = moe.problem(T, K, E, H, I)
    pgu, pd = ops.mx_pack(qgu, True, fmt), ops.mx_pack(qd, False, fmt)
    got, _ = ops.forward_mx(p, x, ids, w, pgu, sgu, pd, sdd, fmt, packed=True)
    fwd = oracle.forward_mxfp8 if fmt == "mxfp8" else oracle.forward_mxfp4
    ref = fwd(bits(x), ids.cpu().numpy(), w.cpu().numpy(), cg, sg, cd, sd)
    check_close(f64(got), ref, f"{fmt} packed {name}")


@pytest.mark.parametrize("name", ["ep_decode_T8", "ep_decode_T32"])
def test_forward_packed_ep_decode_vs_oracle(name):
    cfg = W.CONFIGS[name]
    T, K, E, H, I = cfg.num_tokens, cfg.top_k, cfg.num_experts, cfg.hidden, cfg.intermediate
    x_h = W.make_x(cfg, 2)
    ids_h, w_h = W.make_routing(cfg, 2)
    wgu, wd = W.make_weights(cfg, 2, DEV)
    pgu, pd = ops.skinny_pack(wgu, True), ops.skinny_pack(wd, False)
    p = moe.problem(T, K, E, H, I)
    got, _ = ops.forward_packed(p, x_h.to(DEV), ids_h.to(DEV), w_h.to(DEV), pgu, pd)
    torch.cuda.synchronize()
    del pgu, pd
    ref = oracle.forward(bits(x_h), ids_h.numpy(), w_h.numpy(), DeviceExperts(wgu),
                         DeviceExperts(wd), workers=oracle_workers())
    check_close(f64(got), ref, f"packed {name}")


# ---------------------------------------------------------------------------
# the tiled pack layout (moe_tiled_pack) and the tiled plans on it
# ---------------------------------------------------------------------------
def expected_tiled_pack(w_bits):
    """Written from the layout's definition: per expert, 8-row group g and
    64-value stage s, piece L = row 8g + L/8, k-values 64s + 8c .. +7 with
    c = (L % 8) ^ swz((8g + L/8) % 32)."""
    E, rows, K = w_bits.shape
    G, S = rows // 8, K // 64
    L = np.arange(64)
    r = 8 * np.arange(G)[:, None] + (L // 8)[None, :]                   # [G, 64]
    rm = r % 32
    c = (L % 8)[None, :] ^ (((rm >> 1) & 3) | ((rm >> 2) & 4))          # [G, 64]
    k = 64 * np.arange(S)[None, :, None, None] + 8 * c[:, None, :, None] + np.arange(8)
    out = w_bits[:, r[:, None, :, None], k]                              # [E, G, S, 64, 8]
    return out.reshape(E, rows, K)


@pytest.mark.parametrize("E,rows,K", [(3, 64, 256), (2, 96, 192), (1, 2048, 64), (5, 32, 512)])
def test_tiled_pack_layout(E, rows, K):
    g = torch.Generator().manual_seed(E * rows + K + 1)
    w = torch.randn((E, rows, K), generator=g).to(torch.bfloat16)
    got = ops.tiled_pack(w.to(DEV))
    assert np.array_equal(bits(got), expected_tiled_pack(bits(w)))


TILED_SHAPES = {
    "ragged": (300, 4, 16, 512, 384, -1, 18),
    "i_320": (97, 3, 5, 192, 320, 0, 5),            # gate-up on 128-row weight tiles
    "many_experts_split": (2048, 2, 64, 256, 1024, 0, 64),
    "large_plan": (2016, 2, 4, 512, 1024, 0, 4),    # ~1008 rows per expert: 192 x 256 tiles
}


@pytest.mark.parametrize("name", list(TILED_SHAPES))
@pytest.mark.parametrize("hint", [0, 2, 3, 4])
def test_forward_tiled_packed(name, hint):
    """Bit-identical to moe_forward with the same tiled plan on row-major
    weights, and within the oracle's bar."""
    T, K, E, H, I, lo, hi = TILED_SHAPES[name]
    x, ids, w, wgu, wd = case(T, K, E, H, I, 26, lo, hi)
    p = moe.problem(T, K, E, H, I, 0, hint)
    pgu, pd = ops.tiled_pack(wgu), ops.tiled_pack(wd)
    got, off = ops.forward_tiled_packed(p, x, ids, w, pgu, pd)
    ref_hint = hint if hint else (2 if T * K / E <= 24 else 0)
    ref, ref_off = ops.forward(p if ref_hint == hint else moe.problem(T, K, E, H, I, 0, ref_hint),
                               x, ids, w, wgu, wd)
    assert torch.equal(off, ref_off)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    x_disp, o2, _, _ = ops.dispatch(p, x, ids)
    pr = moe.problem(T, K, E, H, I, 0, ref_hint)
    h_ref = ops.gate_up(pr, x_disp, o2, wgu)
    h = ops.gate_up_tiled_packed(p, x_disp, o2, pgu)
    R = int(o2[-1])
    assert torch.equal(h[:R].view(torch.int16), h_ref[:R].view(torch.int16))
    ids_h = ids.cpu().numpy()
    ref_o = oracle.forward(bits(x), ids_h, w.cpu().numpy(), bits(wgu), bits(wd))
    check_close(f64(got), ref_o, f"tiled packed {name}/hint{hint}")


def test_tiled_packed_refuses_the_skinny_plan():
    T, K, E, H, I, lo, hi = TILED_SHAPES["ragged"]
    x, ids, w, wgu, wd = case(T, K, E, H, I, 27, lo, hi)
    p = moe.problem(T, K, E, H, I, 0, moe.HINT_SKINNY)
    with pytest.raises(moe.MoeError):
        ops.forward_tiled_packed(p, x, ids, w, ops.tiled_pack(wgu), ops.tiled_pack(wd))


@pytest.mark.parametrize("name,seed", [("ep_prefill_T8192", 0), ("ep_prefill_T2048_zipf", 1),
                                       ("mixtral", 0)])
def test_forward_tiled_packed_full_size(name, seed):
    """Full-size prefill and Mixtral-style layers: bit-identical to the
    row-major tiled path (which test_gpu_parity checks against the oracle),
    and 64 covering tokens against the oracle directly."""
    cfg = W.CONFIGS[name]
    T, K, E, H, I = cfg.num_tokens, cfg.top_k, cfg.num_experts, cfg.hidden, cfg.intermediate
    x_h = W.make_x(cfg, seed)
    ids_h, w_h = W.make_routing(cfg, seed)
    wgu, wd = W.make_weights(cfg, seed, DEV)
    p = moe.problem(T, K, E, H, I)
    x, ids, w = x_h.to(DEV), ids_h.to(DEV), w_h.to(DEV)
    ref, _ = ops.forward(p, x, ids, w, wgu, wd)
    pgu = ops.tiled_pack(wgu)
    pd = ops.tiled_pack(wd)
    got, _ = ops.forward_tiled_packed(p, x, ids, w, pgu, pd)
    torch.cuda.synchronize()
    del pgu, pd
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    from helpers import covering_tokens
    toks = covering_tokens(ids_h.numpy(), E, 64, seed=seed)
    r = oracle.forward_tokens(bits(x_h), ids_h.numpy(), w_h.numpy(), DeviceExperts(wgu),
                              DeviceExperts(wd), toks, workers=oracle_workers())
    check_close(f64(got)[toks], r, f"tiled packed {name}")
