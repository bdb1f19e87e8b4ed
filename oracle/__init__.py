"""CPU oracle for the routed-MoE expert path -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding)
never imports, calls or links it, and it shares no code with that path.

What it computes, in float64 from inputs widened exactly from bf16 / fp32:

  For each token t below the valid-token count T_v:
    out[t,:] = sum over j with 0 <= ids[t,j] < E of  w[t,j] * y(ids[t,j], x[t,:])
               (a zero row when no assignment is valid)
    y(e, x)  = W_down[e] @ ( silu(W_gate[e] @ x) * (W_up[e] @ x) )
    W_gate[e] = W_gateup[e, 0:I, :],  W_up[e] = W_gateup[e, I:2I, :]
    silu(z)  = z / (1 + exp(-z))

plus the exact integer dispatch into a tight, unpadded, expert-major batch.

Sources (page title, then section):
  * TileOps PR #1738 "[Refactor][MoE] Separate dispatched expert compute",
    Summary: routed experts = local dispatch -> expert MLP over a tight
    expert-major batch -> combine; routing weights stay outside expert
    compute and are applied in the combine; Scope: BF16 tight/no-pad batches,
    the last entry of expert_offsets is the valid-row count kept on the GPU,
    capacity-tail values are unspecified.  Review follow-up: gate/value
    pointwise epilogue after the gate-up grouped GEMM, then the down GEMM.
  * FlashInfer PR #3980, commit notes on the kernel API migration
    (launch/output): one (tokens, hidden) output with the top-k combine
    reduced inside the layer; Accuracy: checked against a dense fp32 ground
    truth over all experts.

Readings where the pages leave a step open (the plainest one the rest
supports): W_gateup holds the gate rows first and the up rows second
(halves, not interleaved); SiLU is plain (no clamp, bias or scale); weights
are applied after the expert MLP, in the combine; ids outside [0, E) and
tokens at or beyond T_v are dropped; rows of one expert are ordered by the
flattened assignment index a = t*K + j (a stable counting sort).

Pins: every function here is checked by the CPU tests against something
other than itself -- a library dense SwiGLU MLP (E=1, K=1, w=1), a dense
ground truth over all experts built from library matmuls, hand-derived
closed-form values, numpy's stable argsort/bincount for the dispatch, and
invariants (zero input, one-hot weights, linearity, token permutation,
duplicate ids, dropped ids).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_to_f64", "f64_to_bf16_bits", "router_topk", "dispatch", "silu", "expert_mlp",
    "expert_compute", "combine", "forward", "forward_tokens",
]


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64: a bf16 value is
    the upper half of the float32 with the same bits."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v) -> np.ndarray:
    """float64 -> nearest float32 -> bf16 with round-to-nearest-even on the
    dropped 16 bits (NaN kept quiet).  Used only to build test inputs."""
    f = np.ascontiguousarray(v, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16)
    return r


# ---------------------------------------------------------------------------
# Local dispatch (TileOps PR #1738, Summary and Scope)
# ---------------------------------------------------------------------------
def router_topk(logits, top_k: int, num_valid_tokens: int | None = None):
    """Router top-k, the step ahead of dispatch (TileOps PR #1738, Summary:
    the routing weights are produced outside expert compute and carried next
    to the ids).  Reading of the routing the workloads describe: for each
    token t < T_v, the top_k largest of its E logits in decreasing order, equal
    values in increasing expert index, and the softmax over those selected
    values, w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0).

    logits: fp32 [T, E] (widened exactly to float64, so the selection compares
    the very values the GPU compares).  Returns (ids int32 [T_v, K],
    weights float64 [T_v, K])."""
    lg = np.asarray(logits, dtype=np.float64)
    T, E = lg.shape
    tv = T if num_valid_tokens is None else max(0, min(T, int(num_valid_tokens)))
    ids = np.empty((tv, top_k), dtype=np.int32)
    w = np.empty((tv, top_k), dtype=np.float64)
    index = np.arange(E)
    for t in range(tv):
        # lexsort: the last key is the primary one -- value descending, then index
        sel = np.lexsort((index, -lg[t]))[:top_k]
        v = lg[t, sel]
        ex = np.exp(v - v[0])
        ids[t] = sel
        w[t] = ex / ex.sum()
    return ids, w


def dispatch(topk_ids, num_experts: int, num_valid_tokens: int | None = None):
    """Stable counting sort of the routed assignments into a tight,
    expert-major batch.

    topk_ids: int [T, K].  Assignment a = t*K + j is valid iff t < T_v and
    0 <= ids[t,j] < E.

    Returns (counts [E], expert_offsets [E+1], row_src [R], token_row [T*K]):
      counts[e]          number of valid assignments to expert e
      expert_offsets     exclusive prefix sum of counts; expert_offsets[E] = R
                         is the valid-row count
      row_src[r]         the assignment a stored at dispatched row r; within
                         expert e, rows follow increasing a
      token_row[a]       the row of assignment a, or -1 if it is not valid
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, K = ids.shape
    E = int(num_experts)
    tv = T if num_valid_tokens is None else max(0, min(int(num_valid_tokens), T))
    flat = ids.reshape(-1)

    counts = np.zeros(E, dtype=np.int64)
    for a in range(tv * K):                       # histogram
        e = flat[a]
        if 0 <= e < E:
            counts[e] += 1

    offsets = np.zeros(E + 1, dtype=np.int64)     # exclusive scan
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]

    R = int(offsets[E])
    row_src = np.zeros(R, dtype=np.int64)
    token_row = np.full(T * K, -1, dtype=np.int64)
    cursor = offsets[:E].copy()
    for a in range(tv * K):                       # stable scatter, a ascending
        e = flat[a]
        if 0 <= e < E:
            r = cursor[e]
            row_src[r] = a
            token_row[a] = r
            cursor[e] += 1
    return (counts.astype(np.int32), offsets.astype(np.int32),
            row_src.astype(np.int32), token_row.astype(np.int32))


# ---------------------------------------------------------------------------
# Expert MLP (TileOps PR #1738, Summary and Review follow-up)
# ---------------------------------------------------------------------------
def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z)), float64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_mlp(x_rows, w_gateup_e, w_down_e):
    """y = W_down @ (silu(W_gate @ x) * (W_up @ x)) for each row x of x_rows.

    x_rows: float64 [M, H]; w_gateup_e: bf16 bits [2I, H] (gate rows [0,I),
    up rows [I,2I)); w_down_e: bf16 bits [H, I].  Returns float64 [M, H].
    The three matrix products are library matmuls in float64."""
    wgu = bf16_to_f64(w_gateup_e)
    I = wgu.shape[0] // 2
    w_gate, w_up = wgu[:I], wgu[I:]
    w_down = bf16_to_f64(w_down_e)
    x = np.asarray(x_rows, dtype=np.float64)
    g = x @ w_gate.T                              # [M, I]
    u = x @ w_up.T                                # [M, I]
    h = silu(g) * u                               # gated pointwise
    return h @ w_down.T                           # [M, H]


def expert_compute(x_disp, expert_offsets, w_gateup, w_down, rows=None):
    """Dispatched-expert compute on a tight expert-major batch: row r of
    x_disp (bf16 bits [>=R, H]) belongs to the expert e with
    expert_offsets[e] <= r < expert_offsets[e+1].  Returns float64 [R, H] (or
    only the listed rows, in the order given).  Routing weights are not
    involved here."""
    off = np.asarray(expert_offsets, dtype=np.int64)
    E = off.shape[0] - 1
    R = int(off[E])
    want = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    H = w_down.shape[1]
    out = np.zeros((want.shape[0], H), dtype=np.float64)
    owner = np.searchsorted(off, want, side="right") - 1
    for e in range(E):
        sel = np.nonzero(owner == e)[0]
        if sel.size == 0:
            continue
        xr = bf16_to_f64(np.asarray(x_disp)[want[sel]])
        out[sel] = expert_mlp(xr, w_gateup[e], w_down[e])
    return out


# ---------------------------------------------------------------------------
# Weighted top-k combine (TileOps PR #1738 Summary; FlashInfer PR #3980 API notes)
# ---------------------------------------------------------------------------
def combine(y_rows, token_row, topk_weights, num_valid_tokens: int | None = None):
    """out[t,:] = sum_j w[t,j] * y_rows[token_row[t*K+j], :] over the j with a
    valid row (token_row >= 0), for t < T_v; zero rows elsewhere.

    y_rows: float64 [R, H] or bf16 bits (uint16) [R, H].  Returns float64
    [T, H]."""
    w = np.asarray(topk_weights, dtype=np.float32).astype(np.float64)
    T, K = w.shape
    tv = T if num_valid_tokens is None else max(0, min(int(num_valid_tokens), T))
    y = np.asarray(y_rows)
    y = bf16_to_f64(y) if y.dtype == np.uint16 else y.astype(np.float64)
    H = y.shape[1]
    tr = np.asarray(token_row, dtype=np.int64).reshape(T, K)
    out = np.zeros((T, H), dtype=np.float64)
    for t in range(tv):
        for j in range(K):
            r = tr[t, j]
            if r >= 0:
                out[t] += w[t, j] * y[r]
    return out


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------
def forward_tokens(x, topk_ids, topk_weights, w_gateup, w_down, tokens,
                   num_valid_tokens: int | None = None):
    """out[t,:] for the listed tokens only (float64 [len(tokens), H]), straight
    from the definition: sum over the token's valid assignments of
    w[t,j] * y(ids[t,j], x[t]).  x: bf16 bits [T, H]; w_gateup: bf16 bits
    [E, 2I, H]; w_down: bf16 bits [E, H, I] (any object indexable by expert
    that yields such arrays)."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    wts = np.asarray(topk_weights, dtype=np.float32).astype(np.float64)
    T, K = ids.shape
    E = len(w_gateup)
    tv = T if num_valid_tokens is None else max(0, min(int(num_valid_tokens), T))
    toks = np.asarray(tokens, dtype=np.int64)
    H = np.asarray(x).shape[1]
    out = np.zeros((toks.shape[0], H), dtype=np.float64)
    # Group the listed (token, slot) pairs by expert so that each expert's
    # weights are widened once; every product is still one token's own row.
    pairs = {}
    for i, t in enumerate(toks):
        if t >= tv:
            continue
        for j in range(K):
            e = ids[t, j]
            if 0 <= e < E:
                pairs.setdefault(int(e), []).append((i, int(t), j))
    for e, lst in sorted(pairs.items()):
        xr = bf16_to_f64(np.asarray(x)[[t for _, t, _ in lst]])
        y = expert_mlp(xr, np.asarray(w_gateup[e]), np.asarray(w_down[e]))
        for (i, t, j), yrow in zip(lst, y):
            out[i] += wts[t, j] * yrow
    return out


def forward(x, topk_ids, topk_weights, w_gateup, w_down, num_valid_tokens: int | None = None):
    """The whole layer for every token: float64 [T, H]; rows t >= T_v are 0."""
    T = np.asarray(topk_ids).shape[0]
    return forward_tokens(x, topk_ids, topk_weights, w_gateup, w_down, np.arange(T),
                          num_valid_tokens)
