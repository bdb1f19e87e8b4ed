"""Pins of the CPU oracle against things other than itself (no GPU).

Each check is chosen so that a plausible slip in the oracle -- a dropped term,
a swapped gate/up half, a wrong sign in SiLU, a transposed weight, a wrong
assignment index, an unstable dispatch order -- fails at least one of them:

* hand-derived worked examples (dispatch: tests/golden; layer: closed forms
  in terms of silu(1), silu(2), silu(3));
* library routines: numpy's stable argsort / bincount for the dispatch,
  torch's float64 matmul + F.silu for a dense SwiGLU MLP (E=1, K=1, w=1) and
  for a dense ground truth that runs every expert on every token and mixes
  with a routing matrix (the check FlashInfer PR #3980 "Accuracy" describes);
* invariants: zero input, one-hot weights, linearity in the weights, token
  permutation, duplicate ids, dropped ids, the valid-token bound;
* torch's own bf16 conversions for the bit-level helpers.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def rand_bf16(shape, std, gen):
    return (torch.randn(shape, generator=gen, dtype=torch.float32) * std).to(torch.bfloat16)


def rand_problem(T, K, E, H, I, seed, id_lo=0, id_hi=None):
    g = torch.Generator().manual_seed(seed)
    x = rand_bf16((T, H), 1.0, g)
    wgu = rand_bf16((E, 2 * I, H), H ** -0.5, g)
    wd = rand_bf16((E, H, I), I ** -0.5, g)
    hi = E if id_hi is None else id_hi
    ids = torch.randint(id_lo, hi, (T, K), generator=g, dtype=torch.int32)
    w = torch.rand((T, K), generator=g, dtype=torch.float32)
    return x, ids, w, wgu, wd


# ---------------------------------------------------------------------------
# bit-level helpers
# ---------------------------------------------------------------------------
def test_bf16_widen_matches_torch():
    g = torch.Generator().manual_seed(0)
    v = torch.randn(10000, generator=g).to(torch.bfloat16)
    v[:4] = torch.tensor([0.0, -0.0, float("inf"), -float("inf")]).to(torch.bfloat16)
    got = oracle.bf16_to_f64(bits(v))
    ref = v.to(torch.float64).numpy()
    assert np.array_equal(got, ref)
    assert np.signbit(got[1])


def test_bf16_round_matches_torch_rne():
    g = torch.Generator().manual_seed(1)
    f = torch.randn(200000, generator=g, dtype=torch.float64) * 10.0
    # exact ties: bf16 value + half an ulp, in float32
    base = torch.randn(1000, generator=g).to(torch.bfloat16).to(torch.float32)
    ulp_half = base.abs().view(torch.int32).bitwise_and(0x7F800000).view(torch.float32) * 2.0 ** -8
    ties = (base + ulp_half).to(torch.float64)
    f = torch.cat([f, ties])
    ref = bits(f.to(torch.float32).to(torch.bfloat16))
    got = oracle.f64_to_bf16_bits(f.numpy())
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------
# dispatch
# ---------------------------------------------------------------------------
def test_dispatch_worked_example():
    with open(os.path.join(GOLDEN, "dispatch_worked_example.json")) as fh:
        gold = json.load(fh)
    ids = np.array(gold["topk_ids"], dtype=np.int32)
    for case in gold["cases"]:
        c, off, rs, tr = oracle.dispatch(ids, gold["num_experts"], case["num_valid_tokens"])
        assert c.tolist() == case["counts"]
        assert off.tolist() == case["expert_offsets"]
        assert rs.tolist() == case["row_src"]
        assert tr.tolist() == case["token_row"]


@pytest.mark.parametrize("T,K,E,tv,lo,hi,seed", [
    (1, 1, 1, 1, 0, 1, 0), (0, 2, 4, 0, 0, 4, 0), (17, 3, 5, 17, -2, 8, 1),
    (64, 2, 8, 64, 0, 8, 2), (100, 6, 96, 100, 0, 384, 3), (333, 8, 128, 200, 0, 128, 4),
    (50, 4, 3, 7, -5, 5, 5),
])
def test_dispatch_vs_stable_argsort(T, K, E, tv, lo, hi, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(lo, hi, size=(T, K)).astype(np.int32)
    c, off, rs, tr = oracle.dispatch(ids, E, tv)
    flat = ids.reshape(-1).astype(np.int64)
    valid = np.zeros(T * K, dtype=bool)
    valid[: tv * K] = True
    valid &= (flat >= 0) & (flat < E)
    # library: bincount of valid ids, stable argsort with invalid keyed last
    assert np.array_equal(c, np.bincount(flat[valid], minlength=E))
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat[valid], minlength=E))]))
    key = np.where(valid, flat, E)
    order = np.argsort(key, kind="stable")[: int(valid.sum())]
    assert np.array_equal(rs, order)
    inv = np.full(T * K, -1)
    inv[order] = np.arange(order.size)
    assert np.array_equal(tr, inv)
    # invariants
    R = int(off[-1])
    assert R == valid.sum() and np.all(np.diff(off) >= 0)
    assert sorted(rs.tolist()) == sorted(np.nonzero(valid)[0].tolist())
    for e in range(E):
        seg = rs[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(flat[seg] == e)
    assert np.array_equal(tr[rs], np.arange(R))


# ---------------------------------------------------------------------------
# SiLU and the layer: closed forms
# ---------------------------------------------------------------------------
def s(z):
    return z / (1.0 + math.exp(-z))


def test_silu_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 2.0, 40.0, -800.0])
    got = oracle.silu(z)
    assert got[0] == 0.0
    assert got[1] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert got[2] == pytest.approx(-1.0 / (1.0 + math.e), rel=1e-15)
    assert got[3] == pytest.approx(2.0 / (1.0 + math.exp(-2.0)), rel=1e-15)
    assert got[4] == pytest.approx(40.0, rel=1e-15)
    assert got[5] == 0.0


def closed_form_problem():
    """H=2, I=1, E=2, K=2, T=3, every value exact in bf16."""
    wgu = np.array([[[1, 0], [0, 1]],          # expert 0: gate row [1,0], up row [0,1]
                    [[0, 1], [1, 1]]], dtype=np.float64)  # expert 1: gate [0,1], up [1,1]
    wd = np.array([[[1], [2]], [[-1], [0.5]]], dtype=np.float64)  # [E, H, I]
    x = np.array([[1, 2], [0.5, 1], [3, -2]], dtype=np.float64)
    ids = np.array([[0, 1], [1, 1], [0, 7]], dtype=np.int32)
    w = np.array([[0.75, 0.25], [0.5, 0.25], [0.5, 0.5]], dtype=np.float32)
    b = oracle.f64_to_bf16_bits
    return b(x), ids, w, b(wgu), b(wd)


def test_forward_closed_form():
    # Hand derivation (s = silu):
    #  t0: e0 g=1,u=2 -> h=2s(1), y=[2s(1),4s(1)];  e1 g=2,u=3 -> h=3s(2), y=[-3s(2),1.5s(2)]
    #      out0 = .75*y(e0) + .25*y(e1)
    #  t1: e1 twice, g=1,u=1.5 -> h=1.5s(1), y=[-1.5s(1), .75s(1)]; out1 = (.5+.25)*y
    #  t2: e0 g=3,u=-2 -> h=-2s(3), y=[-2s(3),-4s(3)]; id 7 is dropped; out2 = .5*y
    x, ids, w, wgu, wd = closed_form_problem()
    exp = np.array([
        [1.5 * s(1) - 0.75 * s(2), 3.0 * s(1) + 0.375 * s(2)],
        [-1.125 * s(1), 0.5625 * s(1)],
        [-s(3), -2.0 * s(3)],
    ])
    got = oracle.forward(x, ids, w, wgu, wd)
    np.testing.assert_allclose(got, exp, rtol=1e-14, atol=0)
    got2 = oracle.forward(x, ids, w, wgu, wd, num_valid_tokens=2)
    np.testing.assert_allclose(got2[:2], exp[:2], rtol=1e-14, atol=0)
    assert np.all(got2[2] == 0)


# ---------------------------------------------------------------------------
# library cross-checks
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,H,I,seed", [(1, 1, 1, 0), (5, 8, 3, 1), (13, 33, 17, 2), (9, 64, 96, 3)])
def test_dense_swiglu_library(T, H, I, seed):
    x, _, _, wgu, wd = rand_problem(T, 1, 1, H, I, seed)
    ids = torch.zeros((T, 1), dtype=torch.int32)
    w = torch.ones((T, 1), dtype=torch.float32)
    got = oracle.forward(bits(x), ids.numpy(), w.numpy(), bits(wgu), bits(wd))
    X, Wgu, Wd = x.double(), wgu[0].double(), wd[0].double()
    ref = (torch.nn.functional.silu(X @ Wgu[:I].T) * (X @ Wgu[I:].T)) @ Wd.T
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def dense_ground_truth(x, ids, w, wgu, wd, tv=None):
    """Every expert on every token (library bmm + F.silu in float64), mixed by
    a [T, E] routing matrix built with scatter_add."""
    T, K = ids.shape
    E, I2, H = wgu.shape
    I = I2 // 2
    tv = T if tv is None else tv
    X = x.double().unsqueeze(0).expand(E, T, H).contiguous()
    Wg = wgu[:, :I, :].double().transpose(1, 2).contiguous()
    Wu = wgu[:, I:, :].double().transpose(1, 2).contiguous()
    Wd = wd.double().transpose(1, 2).contiguous()
    Y = torch.bmm(torch.nn.functional.silu(torch.bmm(X, Wg)) * torch.bmm(X, Wu), Wd)  # [E, T, H]
    ids64 = ids.long()
    ok = (ids64 >= 0) & (ids64 < E)
    ok[tv:] = False
    C = torch.zeros((T, E + 1), dtype=torch.float64)
    C.scatter_add_(1, torch.where(ok, ids64, torch.full_like(ids64, E)), torch.where(ok, w.double(), torch.zeros_like(w.double())))
    return torch.einsum("te,eth->th", C[:, :E], Y)


@pytest.mark.parametrize("T,K,E,H,I,lo,hi,tv,seed", [
    (7, 2, 3, 16, 8, 0, 3, 7, 0),
    (20, 3, 5, 24, 40, -1, 7, 20, 1),
    (31, 6, 8, 32, 16, 0, 16, 25, 2),
    (64, 2, 8, 256, 512, 0, 8, 64, 3),
])
def test_dense_moe_ground_truth(T, K, E, H, I, lo, hi, tv, seed):
    x, ids, w, wgu, wd = rand_problem(T, K, E, H, I, seed, lo, hi)
    got = oracle.forward(bits(x), ids.numpy(), w.numpy(), bits(wgu), bits(wd), num_valid_tokens=tv)
    ref = dense_ground_truth(x, ids, w, wgu, wd, tv)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
def test_zero_input_and_negative_gate():
    x, ids, w, wgu, wd = rand_problem(16, 2, 4, 32, 16, 7)
    zero = np.zeros_like(bits(x))
    assert np.all(oracle.forward(zero, ids.numpy(), w.numpy(), bits(wgu), bits(wd)) == 0)
    # Gate rows driven far negative: silu -> 0, so out -> 0.  Had the gate and
    # up halves been swapped the output would be far from zero.
    wgu2 = wgu.clone()
    wgu2[:, :16, :] = 0
    wgu2[:, :16, 0] = -1000.0
    xp = x.clone()
    xp[:, 0] = 1.0
    out = oracle.forward(bits(xp), ids.numpy(), w.numpy(), bits(wgu2), bits(wd))
    assert np.abs(out).max() < 1e-300


def test_one_hot_linearity_duplicates_permutation():
    T, K, E, H, I = 12, 3, 4, 24, 20
    x, ids, w, wgu, wd = rand_problem(T, K, E, H, I, 11)
    xb, wgub, wdb, idn, wn = bits(x), bits(wgu), bits(wd), ids.numpy(), w.numpy()
    base = oracle.forward(xb, idn, wn, wgub, wdb)
    # one-hot weights give that expert's MLP output
    oh = np.zeros_like(wn)
    oh[:, 1] = 1.0
    got = oracle.forward(xb, idn, oh, wgub, wdb)
    for t in range(T):
        e = idn[t, 1]
        y = oracle.expert_mlp(oracle.bf16_to_f64(xb[t:t + 1]), wgub[e], wdb[e])
        np.testing.assert_allclose(got[t], y[0], rtol=1e-13, atol=1e-15)
    # linearity: out(a*w1 + w2) = a*out(w1) + out(w2)
    w2 = np.random.default_rng(0).random(wn.shape).astype(np.float32)
    lin = oracle.forward(xb, idn, (wn + w2).astype(np.float32), wgub, wdb)
    expected = base + oracle.forward(xb, idn, w2, wgub, wdb)
    np.testing.assert_allclose(lin, expected, rtol=1e-6, atol=1e-6)
    # duplicates sum: ids [e, e] with (a, b) == id [e] with a + b
    dup = np.array([[2, 2]] * T, dtype=np.int32)
    wd2 = np.array([[0.25, 0.5]] * T, dtype=np.float32)
    one = oracle.forward(xb, dup[:, :1], np.array([[0.75]] * T, dtype=np.float32), wgub, wdb)
    np.testing.assert_allclose(oracle.forward(xb, dup, wd2, wgub, wdb), one, rtol=1e-13, atol=1e-15)
    # token permutation: rows move with their tokens
    perm = np.random.default_rng(1).permutation(T)
    permuted = oracle.forward(xb[perm], idn[perm], wn[perm], wgub, wdb)
    np.testing.assert_allclose(permuted, base[perm], rtol=1e-13, atol=1e-15)
    # dropped ids contribute nothing
    idd = idn.copy()
    idd[:, 0] = E + 3
    wz = wn.copy()
    wz[:, 0] = 0
    np.testing.assert_allclose(oracle.forward(xb, idd, wn, wgub, wdb),
                               oracle.forward(xb, idn, wz, wgub, wdb), rtol=1e-13, atol=1e-15)


def test_stages_compose_to_forward():
    T, K, E, H, I = 40, 2, 8, 64, 48
    x, ids, w, wgu, wd = rand_problem(T, K, E, H, I, 5, -1, 9)
    xb, wgub, wdb, idn, wn = bits(x), bits(wgu), bits(wd), ids.numpy(), w.numpy()
    for tv in (T, 17, 0):
        c, off, rs, tr = oracle.dispatch(idn, E, tv)
        x_disp = xb[rs // K]
        y = oracle.expert_compute(x_disp, off, wgub, wdb)
        out = oracle.combine(y, tr, wn, tv)
        ref = oracle.forward(xb, idn, wn, wgub, wdb, tv)
        np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-15)
        sub = oracle.expert_compute(x_disp, off, wgub, wdb, rows=np.arange(0, int(off[-1]), 3))
        np.testing.assert_allclose(sub, y[::3], rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------------------
# Router top-k
# ---------------------------------------------------------------------------
def _check_router_order(lg, ids, K):
    """Each selected expert beats every unselected one (larger value, or the
    same value and a lower index), the picks are distinct and in decreasing
    order with the same tie rule."""
    T, E = lg.shape
    for t in range(ids.shape[0]):
        sel = [int(e) for e in ids[t]]
        assert len(set(sel)) == K and all(0 <= e < E for e in sel)
        for a, b in zip(sel, sel[1:]):
            assert lg[t, a] > lg[t, b] or (lg[t, a] == lg[t, b] and a < b)
        last = sel[-1]
        for u in set(range(E)) - set(sel):
            assert lg[t, last] > lg[t, u] or (lg[t, last] == lg[t, u] and last < u)


@pytest.mark.parametrize("T,E,K,seed,ties", [(40, 8, 2, 0, False), (30, 96, 6, 1, False),
                                             (20, 64, 64, 2, False), (25, 16, 5, 3, True),
                                             (10, 512, 17, 4, True), (12, 1, 1, 5, False)])
def test_router_order_and_weights(T, E, K, seed, ties):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if ties:                        # many equal values: the index decides
        lg = np.round(lg * 2).astype(np.float32)
    ids, w = oracle.router_topk(lg, K)
    _check_router_order(lg, ids, K)
    # weights: positive, sum to one, ratios exp(l_j - l_0)
    assert np.all(w > 0)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    l64 = lg.astype(np.float64)
    for t in range(T):
        v = l64[t, ids[t]]
        assert np.allclose(w[t] / w[t, 0], np.exp(v - v[0]), rtol=1e-12, atol=0)


def test_router_closed_forms_and_ties():
    # K = 1: weight exactly 1; K = 2: the logistic of the logit gap
    lg = np.array([[0.5, 2.0, -1.0, 2.0], [-0.0, 0.0, -3.0, -3.0]], dtype=np.float32)
    ids, w = oracle.router_topk(lg, 1)
    assert ids.tolist() == [[1], [0]] and np.all(w == 1.0)   # ties: lower index; -0 == +0
    ids, w = oracle.router_topk(lg, 2)
    assert ids.tolist() == [[1, 3], [0, 1]]
    assert np.allclose(w, 0.5, rtol=0, atol=0)
    lg = np.array([[1.0, 3.0, 2.0]], dtype=np.float32)
    ids, w = oracle.router_topk(lg, 2)
    assert ids.tolist() == [[1, 2]]
    assert abs(w[0, 1] - 1.0 / (1.0 + math.exp(1.0))) < 1e-15
    # valid-token bound
    ids, w = oracle.router_topk(np.zeros((5, 4), np.float32), 3, num_valid_tokens=2)
    assert ids.shape == (2, 3) and ids.tolist() == [[0, 1, 2], [0, 1, 2]]


def test_router_matches_generator():
    """The Mixtral-style workload draws its routing as torch.argsort of the
    negated logits (stable) and a torch softmax over the selected ones."""
    import workloads as W
    for name in ("tiny", "mixtral"):
        cfg = W.CONFIGS[name]
        lg = W.make_logits(cfg, 3)
        ids_g, w_g = W.make_routing(cfg, 3)
        ids, w = oracle.router_topk(lg.numpy(), cfg.top_k)
        assert np.array_equal(ids, ids_g.numpy())
        assert np.abs(w - w_g.numpy().astype(np.float64)).max() < 1e-6


@pytest.mark.parametrize("fmt", ["bf16", "mxfp8", "mxfp4"])
def test_thread_pool_changes_nothing(fmt):
    """forward with its per-expert products on a thread pool equals the serial
    evaluation bit for bit (same operands, same accumulation order)."""
    T, K, E, H, I = 40, 3, 6, 64, 64
    xt, idt, wt, wgut, wdt = rand_problem(T, K, E, H, I, 77, -1, E + 1)
    x, ids, w, wgu, wd = bits(xt), idt.numpy(), wt.numpy(), bits(wgut), bits(wdt)
    if fmt == "bf16":
        a = oracle.forward(x, ids, w, wgu, wd, num_valid_tokens=33)
        b = oracle.forward(x, ids, w, wgu, wd, num_valid_tokens=33, workers=4)
    else:
        q = oracle.mxfp8_quantize if fmt == "mxfp8" else oracle.mxfp4_quantize
        f = oracle.forward_mxfp8 if fmt == "mxfp8" else oracle.forward_mxfp4
        cg, sg = q(wgu)
        cd, sd = q(wd)
        a = f(x, ids, w, cg, sg, cd, sd, num_valid_tokens=33)
        b = f(x, ids, w, cg, sg, cd, sd, num_valid_tokens=33, workers=4)
    assert np.array_equal(a.view(np.uint64), b.view(np.uint64))
    assert np.abs(a[:33]).max() > 0 and not a[33:].any()
