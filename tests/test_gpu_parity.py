"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Dispatch results are compared bit for bit; floating-point results to the
bar in helpers.check_close.  Small and ragged shapes run the oracle on every
token, and so do the Mixtral-style layer (seeds 0-2) and the 96-expert decode
shares (T = 1 .. 128, seeds 0-2).  The 96-expert prefill shares (uniform
seeds 0-2, Zipf seeds 0-4) run it on at least 256 tokens chosen to include
every touched expert's first and last dispatched row and the first row of
its last m-tile; the dispatch is checked on every assignment.  Every kernel
plan (skinny split-K, tiled 64, tiled 128, tiled large) is exercised on the
small shapes.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import WidenedExperts, bits, check_close, f64, oracle_workers

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mixture_experts_routed_02_amd as moe
    from mixture_experts_routed_02_amd import ops

DEV = "cuda:0"
HINTS = [1, 2, 3, 4]


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def rand_case(T, K, E, H, I, seed, lo=0, hi=None, dev=DEV):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn((T, H), generator=g)).to(torch.bfloat16)
    wgu = (torch.randn((E, 2 * I, H), generator=g) * H ** -0.5).to(torch.bfloat16)
    wd = (torch.randn((E, H, I), generator=g) * I ** -0.5).to(torch.bfloat16)
    ids = torch.randint(lo, E if hi is None else hi, (T, K), generator=g, dtype=torch.int32)
    w = torch.softmax(torch.randn((T, K), generator=g), dim=1)
    return {"x": x, "topk_ids": ids, "topk_weights": w, "w_gateup": wgu, "w_down": wd}


SMALL = {
    # name: (T, K, E, H, I, id_lo, id_hi)
    "ragged_a": (300, 4, 16, 512, 384, -1, 18),
    "ragged_b": (97, 3, 5, 192, 320, 0, 5),
    "one_expert": (200, 1, 4, 256, 128, 2, 3),
    "sparse_many_experts": (40, 2, 128, 256, 256, 0, 128),
    "single_token": (1, 2, 3, 128, 64, 0, 3),
    # >= 32 experts and >= 2 grids of tiles: the tiled plans split the tile list in two
    "many_experts_split": (2048, 2, 64, 256, 1024, 0, 64),
}


def to_dev(inp):
    return {k: v.to(DEV) for k, v in inp.items()}


def check_dispatch(d_offsets, d_row_src, d_token_row, ids, E, tv):
    c, off, rs, tr = oracle.dispatch(ids.numpy(), E, tv)
    got_off = d_offsets.cpu().numpy()
    assert np.array_equal(got_off, off), (got_off[:8], off[:8])
    R = int(off[-1])
    if d_row_src is not None:
        assert np.array_equal(d_row_src.cpu().numpy()[:R], rs)
    T, K = ids.shape
    n = tv * K
    assert np.array_equal(d_token_row.cpu().numpy()[:n], tr[:n])
    return off, rs, tr


# ---------------------------------------------------------------------------
# dispatch
# ---------------------------------------------------------------------------
DISPATCH_CFGS = ["tiny", "mixtral", "ep_decode_T1", "ep_decode_T8", "ep_decode_T32",
                 "ep_decode_T128", "ep_prefill_T2048", "ep_prefill_T8192",
                 "ep_prefill_T8192_zipf", "static_capacity"]


@pytest.mark.parametrize("name", DISPATCH_CFGS)
@pytest.mark.parametrize("seed", [0, 1])
def test_dispatch_bitexact(name, seed):
    cfg = W.CONFIGS[name]
    x = W.make_x(cfg, seed)
    ids, _ = W.make_routing(cfg, seed)
    p = moe.problem(cfg.num_tokens, cfg.top_k, cfg.num_experts, cfg.hidden, cfg.intermediate,
                    cfg.capacity)
    xd = x.to(DEV)
    x_disp, off, rs, tr = ops.dispatch(p, xd, ids.to(DEV))
    o_off, o_rs, _ = check_dispatch(off, rs, tr, ids, cfg.num_experts, cfg.num_tokens)
    R = int(o_off[-1])
    # x_disp rows are bit copies of x[row_src // K]
    assert torch.equal(x_disp[:R].view(torch.int16).cpu(),
                       x.view(torch.int16)[torch.from_numpy(o_rs // cfg.top_k).long()])


@pytest.mark.parametrize("tv", [0, 1, 37, 2047, 2048, 5000, -3])
def test_dispatch_device_token_count(tv):
    cfg = W.CONFIGS["static_capacity"]
    ids, _ = W.make_routing(cfg, 3)
    x = W.make_x(cfg, 3).to(DEV)
    p = moe.problem(cfg.num_tokens, cfg.top_k, cfg.num_experts, cfg.hidden, cfg.intermediate,
                    cfg.capacity)
    nt = torch.tensor([tv], dtype=torch.int32, device=DEV)
    _, off, rs, tr = ops.dispatch(p, x, ids.to(DEV), num_tokens_dev=nt)
    tv_eff = max(0, min(tv, cfg.num_tokens))
    check_dispatch(off, rs, tr, ids, cfg.num_experts, tv_eff)
    # assignments past T_v are marked dropped
    assert bool((tr[tv_eff * cfg.top_k:] == -1).all())


@pytest.mark.parametrize("case", ["all_one_expert", "all_invalid", "one_expert_total",
                                  "duplicates", "max_experts", "multi_block_skew", "empty"])
def test_dispatch_edges(case):
    g = torch.Generator().manual_seed(5)
    if case == "all_one_expert":
        T, K, E = 3000, 4, 64
        ids = torch.full((T, K), 17, dtype=torch.int32)
    elif case == "all_invalid":
        T, K, E = 500, 6, 96
        ids = torch.randint(96, 400, (T, K), generator=g, dtype=torch.int32)
        ids[::2] = -ids[::2]
    elif case == "one_expert_total":
        T, K, E = 777, 2, 1
        ids = torch.randint(-1, 2, (T, K), generator=g, dtype=torch.int32)
    elif case == "duplicates":
        T, K, E = 64, 8, 4
        ids = torch.randint(0, 4, (T, K), generator=g, dtype=torch.int32)
    elif case == "max_experts":
        T, K, E = 4000, 8, 512
        ids = torch.randint(0, 512, (T, K), generator=g, dtype=torch.int32)
    elif case == "multi_block_skew":
        T, K, E = 20000, 3, 7
        ids = torch.randint(0, 7, (T, K), generator=g, dtype=torch.int32)
        ids[: T // 2] = 3
    else:
        T, K, E = 0, 2, 4
        ids = torch.zeros((0, K), dtype=torch.int32)
    H = 64
    x = torch.randn((T, H), generator=g).to(torch.bfloat16)
    p = moe.problem(T, K, E, H, 64)
    x_disp, off, rs, tr = ops.dispatch(p, x.to(DEV), ids.to(DEV))
    o_off, o_rs, _ = check_dispatch(off, rs, tr, ids, E, T)
    R = int(o_off[-1])
    if R:
        assert torch.equal(x_disp[:R].view(torch.int16).cpu(),
                           x.view(torch.int16)[torch.from_numpy(o_rs // K).long()])


@pytest.mark.parametrize("T,K,E,skew,tv", [
    (1 << 19, 8, 128, False, None),          # T*K = 2^22: 1024 dispatch blocks
    (1 << 19, 8, 128, False, 300001),        # device token count mid-block
    (1 << 20, 4, 512, True, None),           # 2^22 over 512 experts, three hold half of them
])
def test_dispatch_many_blocks(T, K, E, skew, tv):
    """The multi-block dispatch far past the five workloads' sizes: 1024
    blocks, whose per-block histograms are scanned over the blocks by a
    separate kernel, bit-exact against the oracle."""
    g = torch.Generator().manual_seed(T + E)
    ids = torch.randint(-1, E + 2, (T, K), generator=g, dtype=torch.int32)
    if skew:
        hot = torch.randint(0, 3, (T, K), generator=g, dtype=torch.int32) + 200
        ids = torch.where(torch.rand((T, K), generator=g) < 0.5, hot, ids)
    p = moe.problem(T, K, E, 64, 64)
    x = torch.zeros((T, 64), dtype=torch.bfloat16, device=DEV)
    nt = None if tv is None else torch.tensor([tv], dtype=torch.int32, device=DEV)
    _, off, rs, tr = ops.dispatch(p, x, ids.to(DEV), num_tokens_dev=nt)
    tvv = T if tv is None else tv
    check_dispatch(off, rs, tr, ids, E, tvv)
    assert bool((tr[tvv * K:] == -1).all())


# ---------------------------------------------------------------------------
# combine
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,K,E,H,lo,hi,tv", [
    (64, 2, 8, 256, 0, 8, 64), (333, 6, 96, 7168, 0, 384, 333), (2048, 8, 128, 2048, 0, 128, 1234),
    (5, 3, 2, 64, -2, 4, 5),
])
def test_combine_vs_oracle(T, K, E, H, lo, hi, tv):
    g = torch.Generator().manual_seed(T)
    ids = torch.randint(lo, hi, (T, K), generator=g, dtype=torch.int32)
    w = torch.rand((T, K), generator=g)
    _, off, rs, tr = oracle.dispatch(ids.numpy(), E, tv)
    cap = T * K
    y = W.make_bf16_rows(cap, H, seed=T)
    p = moe.problem(T, K, E, H, 64)
    out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=DEV)
    nt = torch.tensor([tv], dtype=torch.int32, device=DEV)
    tr_full = np.full(T * K, -1, dtype=np.int32)
    tr_full[: tv * K] = tr[: tv * K]
    ops.combine(p, y.to(DEV), torch.from_numpy(tr_full).to(DEV), w.to(DEV), num_tokens_dev=nt,
                out=out)
    ref = oracle.combine(bits(y), tr_full, w.numpy(), tv)
    got = f64(out)
    # out is one bf16 rounding of an fp32 sum: within half an ulp plus fp32 error
    err = np.abs(got[:tv] - ref[:tv])
    assert np.all(err <= 2.0 ** -8 * np.abs(ref[:tv]) + 1e-6 * np.abs(ref).max()), err.max()
    assert np.all(np.isnan(got[tv:]))   # rows past T_v untouched
    no_valid = np.all(tr_full.reshape(T, K)[:tv] < 0, axis=1)
    assert np.all(got[:tv][no_valid] == 0)


# ---------------------------------------------------------------------------
# expert compute and the whole layer on small / ragged shapes (full oracle)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("hint", HINTS)
def test_expert_compute_small(name, hint):
    T, K, E, H, I, lo, hi = SMALL[name]
    inp = rand_case(T, K, E, H, I, seed=11, lo=lo, hi=hi)
    _, off, rs, _ = oracle.dispatch(inp["topk_ids"].numpy(), E, T)
    R = int(off[-1])
    cap = T * K
    xb = bits(inp["x"])
    x_disp = np.zeros((cap, H), dtype=np.uint16)
    x_disp[:R] = xb[rs // K]
    p = moe.problem(T, K, E, H, I, 0, hint)
    d_xd = torch.from_numpy(x_disp.view(np.int16)).view(torch.bfloat16).to(DEV)
    d_off = torch.from_numpy(off).to(DEV)
    y = torch.full((cap, H), float("nan"), dtype=torch.bfloat16, device=DEV)
    ops.expert_compute(p, d_xd, d_off, inp["w_gateup"].to(DEV), inp["w_down"].to(DEV), y_disp=y)
    ref = oracle.expert_compute(x_disp, off, bits(inp["w_gateup"]), bits(inp["w_down"]))
    check_close(f64(y[:R]), ref, f"{name}/hint{hint}")


@pytest.mark.parametrize("name", list(SMALL) + ["tiny"])
@pytest.mark.parametrize("hint", [0] + HINTS)
def test_forward_small(name, hint):
    if name == "tiny":
        cfg = W.CONFIGS["tiny"]
        inp = W.make_inputs(cfg, 0)
        T, K, E, H, I = cfg.num_tokens, cfg.top_k, cfg.num_experts, cfg.hidden, cfg.intermediate
    else:
        T, K, E, H, I, lo, hi = SMALL[name]
        inp = rand_case(T, K, E, H, I, seed=12, lo=lo, hi=hi)
    d = to_dev(inp)
    p = moe.problem(T, K, E, H, I, 0, hint)
    out, off = ops.forward(p, d["x"], d["topk_ids"], d["topk_weights"], d["w_gateup"], d["w_down"])
    ref = oracle.forward(bits(inp["x"]), inp["topk_ids"].numpy(), inp["topk_weights"].numpy(),
                         bits(inp["w_gateup"]), bits(inp["w_down"]))
    _, o_off, _, _ = oracle.dispatch(inp["topk_ids"].numpy(), E, T)
    assert np.array_equal(off.cpu().numpy(), o_off)
    check_close(f64(out), ref, f"{name}/hint{hint}")


@pytest.mark.parametrize("seed", [1, 2])
def test_forward_tiny_seeds(seed):
    cfg = W.CONFIGS["tiny"]
    inp = W.make_inputs(cfg, seed)
    d = to_dev(inp)
    p = moe.problem(cfg.num_tokens, cfg.top_k, cfg.num_experts, cfg.hidden, cfg.intermediate)
    out, off = ops.forward(p, d["x"], d["topk_ids"], d["topk_weights"], d["w_gateup"], d["w_down"])
    ref = oracle.forward(bits(inp["x"]), inp["topk_ids"].numpy(), inp["topk_weights"].numpy(),
                         bits(inp["w_gateup"]), bits(inp["w_down"]))
    check_close(f64(out), ref, f"tiny seed {seed}")


# ---------------------------------------------------------------------------
# full-size workloads, sampled tokens
# ---------------------------------------------------------------------------
_weights_cache = {}


def device_weights(cfg, seed):
    key = (cfg.num_experts, cfg.hidden, cfg.intermediate, seed)
    if key not in _weights_cache:
        _weights_cache.clear()
        torch.cuda.empty_cache()
        _weights_cache[key] = W.make_weights(cfg, seed, DEV)
    return _weights_cache[key]


def run_full_size(name, seed, weights=None):
    """One moe_forward of a full-size workload: x and routing of `seed`, the
    given device weights (else those of `seed`).  Returns (cfg, host x, ids,
    w, out)."""
    cfg = W.CONFIGS[name]
    wgu, wd = weights if weights is not None else device_weights(cfg, seed)
    x = W.make_x(cfg, seed)
    ids, w = W.make_routing(cfg, seed)
    p = moe.problem(cfg.num_tokens, cfg.top_k, cfg.num_experts, cfg.hidden, cfg.intermediate)
    print(f"[full] {name} seed {seed}", flush=True)
    out, off = ops.forward(p, x.to(DEV), ids.to(DEV), w.to(DEV), wgu, wd)
    torch.cuda.synchronize()
    _, o_off, _, _ = oracle.dispatch(ids.numpy(), cfg.num_experts, cfg.num_tokens)
    assert np.array_equal(off.cpu().numpy(), o_off)
    return cfg, x, ids, w, out


def check_tokens(name, seed, cfg, x, ids, w, widen, out, toks, workers):
    ref = oracle.forward_tokens_widened(bits(x), ids.numpy(), w.numpy(), cfg.num_experts, widen,
                                        toks, workers=workers)
    got = f64(out)[toks]
    fro, mx = check_close(got, ref, f"{name} seed {seed}")
    print(f"[full] {name} seed {seed}: {len(toks)} tokens, rel_fro={fro:.2e} max_rel={mx:.2e}",
          flush=True)
    # tokens with no local expert produce exact zeros
    local = ((ids >= 0) & (ids < cfg.num_experts)).any(dim=1).numpy()
    assert np.all(f64(out)[~local] == 0)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_forward_mixtral_every_token(seed):
    """The Mixtral-style layer (~1024 ragged rows per expert: the branch-free
    192 x 256 tiled instances) against the oracle on all 4096 tokens."""
    cfg = W.CONFIGS["mixtral"]
    wgu, wd = device_weights(cfg, seed)
    cfg, x, ids, w, out = run_full_size("mixtral", seed, (wgu, wd))
    check_tokens("mixtral", seed, cfg, x, ids, w, WidenedExperts(wgu, wd), out,
                 np.arange(cfg.num_tokens), 1)


@pytest.fixture(scope="module")
def ep_share():
    """The 96-expert, 7168 x 3072 expert-parallel share's weights (seed 0,
    drawn on the device) and a cache of their widened host copies, shared by
    every decode and prefill case below (x and routing vary by seed)."""
    _weights_cache.clear()
    torch.cuda.empty_cache()
    wgu, wd = W.make_weights(W.CONFIGS["ep_prefill_T8192"], 0, DEV)
    yield wgu, wd, WidenedExperts(wgu, wd)
    del wgu, wd
    torch.cuda.empty_cache()


DECODE = ["ep_decode_T1", "ep_decode_T8", "ep_decode_T32", "ep_decode_T128"]


@pytest.mark.parametrize("name", DECODE)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_forward_ep_decode_every_token(name, seed, ep_share):
    wgu, wd, widen = ep_share
    cfg, x, ids, w, out = run_full_size(name, seed, (wgu, wd))
    check_tokens(name, seed, cfg, x, ids, w, widen, out, np.arange(cfg.num_tokens),
                 oracle_workers())


PREFILL = [(n, s) for n in ("ep_prefill_T2048", "ep_prefill_T8192") for s in (0, 1, 2)] + \
          [(n, s) for n in ("ep_prefill_T2048_zipf", "ep_prefill_T8192_zipf") for s in range(5)] + \
          [("ep_prefill_T16384", 0)]


@pytest.mark.parametrize("name,seed", PREFILL)
def test_forward_ep_prefill_every_token(name, seed, ep_share):
    """96-of-384 prefill (uniform seeds 0-2, Zipf s = 1.2 seeds 0-4, 2048 and
    8192 tokens, and the 16384-token point) on every token against the
    oracle; the Zipf layers include local experts with up to 37 m-tiles."""
    wgu, wd, widen = ep_share
    cfg, x, ids, w, out = run_full_size(name, seed, (wgu, wd))
    check_tokens(name, seed, cfg, x, ids, w, widen, out, np.arange(cfg.num_tokens),
                 oracle_workers())


# ---------------------------------------------------------------------------
# static capacity + graph replay
# ---------------------------------------------------------------------------
def test_static_capacity_graph_replays():
    cfg = W.CONFIGS["static_capacity"]
    T, K, E, H, I = cfg.num_tokens, cfg.top_k, cfg.num_experts, cfg.hidden, cfg.intermediate
    wgu, wd = device_weights(cfg, 0)
    p = moe.problem(T, K, E, H, I, cfg.capacity)
    x_buf = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    ids_buf = torch.zeros((T, K), dtype=torch.int32, device=DEV)
    w_buf = torch.zeros((T, K), dtype=torch.float32, device=DEV)
    nt = torch.zeros((1,), dtype=torch.int32, device=DEV)
    graph = ops.MoEGraph(p, x_buf, ids_buf, w_buf, wgu, wd, num_tokens_dev=nt)
    tvs = W.make_static_token_counts(0)
    ex_off = torch.empty((E + 1,), dtype=torch.int32, device=DEV)
    ex_out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    ws = ops.make_workspace(p, DEV)
    widen = WidenedExperts(wgu, wd)
    for i, tv in enumerate(tvs):
        x = W.make_x(cfg, 100 + i)
        ids, w = W.make_routing(cfg, 100 + i)
        x_buf.copy_(x)
        ids_buf.copy_(ids)
        w_buf.copy_(w)
        nt.fill_(tv)
        graph.out.view(torch.int16).fill_(0x7FC1)    # a NaN pattern no kernel writes
        graph.launch()
        torch.cuda.synchronize()
        _, o_off, _, _ = oracle.dispatch(ids.numpy(), E, tv)
        assert np.array_equal(graph.expert_offsets.cpu().numpy(), o_off), f"replay {i} T_v={tv}"
        got = graph.out.clone()
        # rows past T_v are untouched
        assert bool((got[tv:].view(torch.int16) == 0x7FC1).all()), f"replay {i}"
        toks = np.arange(tv)                           # every valid token
        ref = oracle.forward_tokens_widened(bits(x), ids.numpy(), w.numpy(), E, widen, toks,
                                            num_valid_tokens=tv, workers=oracle_workers())
        check_close(f64(got)[toks], ref, f"replay {i} T_v={tv}")
        # the graph replays exactly what an eager call computes
        ops.forward(p, x_buf, ids_buf, w_buf, wgu, wd, num_tokens_dev=nt, expert_offsets=ex_off,
                    out=ex_out, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(ex_out[:tv].view(torch.int16), got[:tv].view(torch.int16)), f"replay {i}"
    graph.close()


# ---------------------------------------------------------------------------
# properties that hold at any size
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("hint", HINTS)
def test_properties(hint):
    T, K, E, H, I = 300, 4, 16, 512, 384
    inp = rand_case(T, K, E, H, I, seed=21, lo=-1, hi=18)
    d = to_dev(inp)
    p = moe.problem(T, K, E, H, I, 0, hint)
    ws = ops.make_workspace(p, DEV)
    ws.view(torch.int16).fill_(-1)                     # NaN bit patterns everywhere
    out1, off1 = ops.forward(p, d["x"], d["topk_ids"], d["topk_weights"], d["w_gateup"],
                             d["w_down"], workspace=ws)
    out1 = out1.clone()
    # repeated calls are bit-identical (nothing accumulates in the workspace)
    out2, _ = ops.forward(p, d["x"], d["topk_ids"], d["topk_weights"], d["w_gateup"],
                          d["w_down"], workspace=ws)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert bool(torch.isfinite(out1.float()).all())
    # the three stages compose to the fused call bit for bit
    x_disp, off, rs, tr = ops.dispatch(p, d["x"], d["topk_ids"])
    y = ops.expert_compute(p, x_disp, off, d["w_gateup"], d["w_down"])
    out3 = ops.combine(p, y, tr, d["topk_weights"])
    assert torch.equal(out1.view(torch.int16), out3.view(torch.int16))
    h = ops.gate_up(p, x_disp, off, d["w_gateup"])
    y2 = ops.down(p, h, off, d["w_down"])
    R = int(off[-1])
    assert torch.equal(y[:R].view(torch.int16), y2[:R].view(torch.int16))
    # token permutation moves rows bit-identically
    perm = torch.randperm(T, generator=torch.Generator().manual_seed(3))
    outp, _ = ops.forward(p, d["x"][perm.to(DEV)].contiguous(), d["topk_ids"][perm.to(DEV)].contiguous(),
                          d["topk_weights"][perm.to(DEV)].contiguous(), d["w_gateup"], d["w_down"])
    assert torch.equal(outp.view(torch.int16), out1[perm.to(DEV)].view(torch.int16))
    # linearity in the routing weights (within bf16 rounding of out)
    out4, _ = ops.forward(p, d["x"], d["topk_ids"], (d["topk_weights"] * 0.5).contiguous(),
                          d["w_gateup"], d["w_down"])
    check_close(f64(out4) * 2.0, f64(out1), "linearity")
    # zero input gives an exactly zero output
    outz, _ = ops.forward(p, torch.zeros_like(d["x"]), d["topk_ids"], d["topk_weights"],
                          d["w_gateup"], d["w_down"])
    assert bool((outz.float() == 0).all())
    # gate rows driven far negative: silu -> 0, so the output is 0 (pins gate/up order)
    wgu2 = d["w_gateup"].clone()
    wgu2[:, :I, :] = 0
    wgu2[:, :I, 0] = -1000.0
    x2 = d["x"].clone()
    x2[:, 0] = 1.0
    outn, _ = ops.forward(p, x2, d["topk_ids"], d["topk_weights"], wgu2, d["w_down"])
    assert float(outn.float().abs().max()) == 0.0


def test_zero_tokens():
    p = moe.problem(0, 2, 8, 256, 512)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    ids = torch.empty((0, 2), dtype=torch.int32, device=DEV)
    w = torch.empty((0, 2), dtype=torch.float32, device=DEV)
    wgu = torch.zeros((8, 1024, 256), dtype=torch.bfloat16, device=DEV)
    wd = torch.zeros((8, 256, 512), dtype=torch.bfloat16, device=DEV)
    out, off = ops.forward(p, x, ids, w, wgu, wd)
    assert out.shape == (0, 256)
    assert bool((off == 0).all())


@pytest.mark.parametrize("T,K,E,H,I,lo,hi,tv", [
    (1, 6, 96, 512, 256, 0, 384, None),      # one token, most ids non-local
    (37, 6, 16, 256, 192, -1, 20, None),
    (170, 6, 8, 128, 128, 0, 8, 101),        # T*K = 1020, device-side T_v
    (5, 2, 4, 64, 64, 7, 9, None),           # no valid assignment at all
    # T*K <= 8 and I % 1024 == 0: the down kernel also does the combine
    (1, 6, 96, 256, 1024, 0, 384, None),
    (2, 4, 8, 128, 1024, 0, 8, None),        # duplicates likely: 8 rows over 8 experts
    (4, 2, 8, 64, 1024, 0, 8, 3),            # device-side T_v
    (1, 6, 8, 64, 1024, 9, 12, None),        # every id dropped: a zero row
])
def test_small_batch_forward_composes(T, K, E, H, I, lo, hi, tv):
    """moe_forward on a small batch (T*K <= 1024, skinny plan: the gate-up
    kernel does the dispatch itself) equals the staged calls bit for bit and
    the oracle to tolerance, on two calls in a row with one workspace.
    Outputs start as a NaN sentinel: rows t < T_v must be written (zero rows
    when nothing is valid), rows t >= T_v are left alone by both paths."""
    inp = rand_case(T, K, E, H, I, seed=31, lo=lo, hi=hi)
    d = to_dev(inp)
    p = moe.problem(T, K, E, H, I, 0, 1)
    nt = None if tv is None else torch.tensor([tv], dtype=torch.int32, device=DEV)

    def sentinel():
        o = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
        o.view(torch.int16).fill_(0x7FC1)
        return o

    x_disp, off2, rs, tr = ops.dispatch(p, d["x"], d["topk_ids"], num_tokens_dev=nt)
    y = ops.expert_compute(p, x_disp, off2, d["w_gateup"], d["w_down"])
    out2 = ops.combine(p, y, tr, d["topk_weights"], num_tokens_dev=nt, out=sentinel())
    ws = ops.make_workspace(p, DEV)
    for call in range(2):
        out, off = ops.forward(p, d["x"], d["topk_ids"], d["topk_weights"], d["w_gateup"],
                               d["w_down"], num_tokens_dev=nt, out=sentinel(), workspace=ws)
        assert torch.equal(off, off2), f"call {call}"
        assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), f"call {call}"
    tvv = T if tv is None else tv
    ref = oracle.forward(bits(inp["x"]), inp["topk_ids"].numpy(), inp["topk_weights"].numpy(),
                         bits(inp["w_gateup"]), bits(inp["w_down"]), num_valid_tokens=tvv)
    _, o_off, _, _ = oracle.dispatch(inp["topk_ids"].numpy(), E, tvv)
    assert np.array_equal(off.cpu().numpy(), o_off)
    check_close(f64(out)[:tvv], ref[:tvv], f"small batch T={T}")
