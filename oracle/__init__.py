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
    "expert_mlp_f64",
    "expert_compute", "combine", "forward", "forward_tokens", "forward_tokens_widened",
    "e4m3_to_f64", "e8m0_to_f64", "mxfp8_quantize", "mxfp8_to_f64",
    "forward_tokens_mxfp8", "forward_mxfp8", "e2m1_to_f64", "mxfp4_quantize", "mxfp4_to_f64",
    "forward_tokens_mxfp4", "forward_mxfp4",
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
    return expert_mlp_f64(x_rows, bf16_to_f64(w_gateup_e), bf16_to_f64(w_down_e))


def expert_mlp_f64(x_rows, wgu, w_down):
    """expert_mlp on weights already widened to float64 (wgu [2I, H], gate
    rows first; w_down [H, I])."""
    I = wgu.shape[0] // 2
    w_gate, w_up = wgu[:I], wgu[I:]
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
                   num_valid_tokens: int | None = None, workers: int = 1):
    """out[t,:] for the listed tokens only (float64 [len(tokens), H]), straight
    from the definition: sum over the token's valid assignments of
    w[t,j] * y(ids[t,j], x[t]).  x: bf16 bits [T, H]; w_gateup: bf16 bits
    [E, 2I, H]; w_down: bf16 bits [E, H, I] (any object indexable by expert
    that yields such arrays).  workers > 1 evaluates the experts' MLPs on that
    many threads; the result is the same to the bit (see
    forward_tokens_widened)."""
    return forward_tokens_widened(
        x, topk_ids, topk_weights, len(w_gateup),
        lambda e: (bf16_to_f64(np.asarray(w_gateup[e])), bf16_to_f64(np.asarray(w_down[e]))),
        tokens, num_valid_tokens, workers)


def forward_tokens_widened(x, topk_ids, topk_weights, E, widen, tokens,
                           num_valid_tokens: int | None = None, workers: int = 1):
    """forward_tokens with the expert weights supplied as float64 by
    widen(e) -> (W_gateup[e] [2I, H], W_down[e] [H, I]) (for instance the
    exact widening bf16_to_f64 of the bf16 weights, computed once and reused
    across calls).

    workers only changes where the per-expert products run: each expert's
    y rows are the same library calls on the same operands either way, and
    they are added into out in the same (increasing expert) order, so the
    result does not depend on it."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    wts = np.asarray(topk_weights, dtype=np.float32).astype(np.float64)
    T, K = ids.shape
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
    items = sorted(pairs.items())

    def expert_rows(item):
        e, lst = item
        xr = bf16_to_f64(np.asarray(x)[[t for _, t, _ in lst]])
        return expert_mlp_f64(xr, *widen(e))

    if workers > 1 and len(items) > 1:
        import contextlib
        from concurrent.futures import ThreadPoolExecutor
        try:
            from threadpoolctl import threadpool_limits
            one_blas_thread = threadpool_limits(1)
        except ImportError:  # pragma: no cover
            one_blas_thread = contextlib.nullcontext()
        # one BLAS thread per worker: the per-expert products are small, and a
        # BLAS thread pool per worker oversubscribes the cores many times over
        with one_blas_thread, ThreadPoolExecutor(max_workers=workers) as pool:
            ys = list(pool.map(expert_rows, items))
    else:
        ys = [expert_rows(it) for it in items]
    for (e, lst), y in zip(items, ys):
        for (i, t, j), yrow in zip(lst, y):
            out[i] += wts[t, j] * yrow
    return out


def forward(x, topk_ids, topk_weights, w_gateup, w_down, num_valid_tokens: int | None = None,
            workers: int = 1):
    """The whole layer for every token: float64 [T, H]; rows t >= T_v are 0."""
    T = np.asarray(topk_ids).shape[0]
    return forward_tokens(x, topk_ids, topk_weights, w_gateup, w_down, np.arange(T),
                          num_valid_tokens, workers)


# ---------------------------------------------------------------------------
# MXFP8 expert weights (FlashInfer PR #3980: the MXFP8 MegaMoE backend, and
# the commit notes on the quantized combine wire, whose 'mxfp8' format is
# blocks of 32 e4m3 values sharing one e8m0 scale).  TileOps PR #1738 Scope
# leaves FP8 outside the BF16 path; this is the low-precision weight variant
# of the same layer.
#
# Readings (the pages name the format, not the recipe):
#   * e4m3 is the OCP FP8 E4M3 ("fn") encoding: sign, 4 exponent bits with
#     bias 7, 3 mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6;
#     S.1111.111 is NaN; there are no infinities; the largest value is 448.
#   * e8m0 is a bare biased exponent: code s means 2^(s - 127) (255 = NaN).
#   * one scale per 32 consecutive values along K (the contraction axis) of
#     every weight row.
#   * the scale of a block is 2^(floor(log2(amax)) - 8), 8 being the exponent
#     of e4m3's largest binade (the OCP MX recipe), with the code clamped to
#     [0, 254]; an all-zero block takes code 0.
#   * elements are v / scale rounded to the nearest e4m3 value, ties to even
#     mantissa, magnitudes above 448 saturated to 448; the sign bit of the
#     code is the sign bit of the input (so -0 stays -0).
#   * the layer computes with the dequantized weights q * scale (exact in
#     float64); the activations stay bf16.
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0
MX_BLOCK = 32


def _e4m3_value(c: np.ndarray) -> np.ndarray:
    """The E4M3 encoding written out: sign, exponent field, mantissa field."""
    c = c.astype(np.int64)
    sign = (c >> 7) & 1
    ex = (c >> 3) & 15
    man = c & 7
    mag = np.where(ex == 0, man / 8.0 * 2.0 ** -6, (1.0 + man / 8.0) * np.exp2(ex - 7.0))
    v = np.where(sign == 1, -mag, mag)
    return np.where((ex == 15) & (man == 7), np.nan, v)


_E4M3_VALUES = _e4m3_value(np.arange(256))


def e4m3_to_f64(codes) -> np.ndarray:
    """Value of OCP FP8 E4M3 codes (uint8) as float64 (the 256 values of the
    encoding, looked up by code)."""
    return _E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e8m0_to_f64(codes) -> np.ndarray:
    """Value of E8M0 scale codes (uint8): 2^(s - 127), NaN for 255."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def _round_to_e4m3(y: np.ndarray) -> np.ndarray:
    """Nearest e4m3 magnitude to |y| (float64, exact), ties to even mantissa,
    saturated at 448.  Normal binades [2^E, 2^(E+1)) hold 8 values spaced
    2^(E-3); below 2^-6 the spacing is the subnormal step 2^-9."""
    a = np.abs(y)
    _, ex = np.frexp(a)                     # a = f * 2^ex, f in [0.5, 1)
    binade = np.maximum(ex - 1, -6)         # floor(log2 a), subnormals share -6's step
    step = np.exp2(binade - 3.0)
    q = np.round(a / step) * step           # np.round: half to even
    return np.minimum(q, E4M3_MAX)


def _encode_e4m3(mag: np.ndarray, sign: np.ndarray) -> np.ndarray:
    """Code of an exactly representable e4m3 magnitude (<= 448) and a sign."""
    code = np.zeros(mag.shape, dtype=np.int64)
    sub = mag < 2.0 ** -6
    code[sub] = np.rint(mag[sub] / 2.0 ** -9).astype(np.int64)        # exponent field 0
    f, ex = np.frexp(mag[~sub])
    e_field = (ex - 1) + 7
    m_field = np.rint((f * 2.0 - 1.0) * 8.0).astype(np.int64)
    code[~sub] = (e_field << 3) | m_field
    return (code | (sign.astype(np.int64) << 7)).astype(np.uint8)


def mxfp8_quantize(w_bits):
    """MXFP8 quantization of bf16 weights along their last axis.

    w_bits: bf16 bits (uint16) [..., K], K a multiple of 32.  Returns
    (codes uint8 [..., K], scales uint8 [..., K // 32]) with
    value(codes[..., k]) * 2^(scales[..., k // 32] - 127) the dequantized
    weight."""
    b = np.ascontiguousarray(w_bits, dtype=np.uint16)
    K = b.shape[-1]
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    v = bf16_to_f64(b).reshape(b.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    amax = np.abs(v).max(axis=-1)
    _, ex = np.frexp(amax)                                   # amax = f * 2^ex
    s_code = np.where(amax > 0, np.clip((ex - 1) - 8 + 127, 0, 254), 0).astype(np.int64)
    y = v / np.exp2(s_code - 127.0)[..., None]               # exact: power-of-two scale
    mag = _round_to_e4m3(y)
    sign = (b.reshape(v.shape) >> np.uint16(15)).astype(np.int64)
    codes = _encode_e4m3(mag, sign).reshape(b.shape)
    return codes, s_code.astype(np.uint8)


def mxfp8_to_f64(codes, scales) -> np.ndarray:
    """Dequantized MXFP8 weights: e4m3 value times its block's e8m0 scale."""
    c = np.asarray(codes, dtype=np.uint8)
    s = np.asarray(scales, dtype=np.uint8)
    K = c.shape[-1]
    return e4m3_to_f64(c) * np.repeat(e8m0_to_f64(s), MX_BLOCK, axis=-1)[..., :K]


def forward_tokens_mxfp8(x, topk_ids, topk_weights, wgu_codes, wgu_scales, wd_codes, wd_scales,
                         tokens, num_valid_tokens: int | None = None, workers: int = 1):
    """forward_tokens with MXFP8 expert weights: codes [E, 2I, H] / scales
    [E, 2I, H/32] for W_gateup, codes [E, H, I] / scales [E, H, I/32] for
    W_down (any objects indexable by expert), dequantized exactly to float64
    and then the same layer definition."""
    return forward_tokens_widened(
        x, topk_ids, topk_weights, len(wgu_codes),
        lambda e: (mxfp8_to_f64(wgu_codes[e], wgu_scales[e]), mxfp8_to_f64(wd_codes[e], wd_scales[e])),
        tokens, num_valid_tokens, workers)


def forward_mxfp8(x, topk_ids, topk_weights, wgu_codes, wgu_scales, wd_codes, wd_scales,
                  num_valid_tokens: int | None = None, workers: int = 1):
    """The whole MXFP8-weight layer for every token: float64 [T, H]."""
    T = np.asarray(topk_ids).shape[0]
    return forward_tokens_mxfp8(x, topk_ids, topk_weights, wgu_codes, wgu_scales, wd_codes,
                                wd_scales, np.arange(T), num_valid_tokens, workers)


# ---------------------------------------------------------------------------
# MXFP4 expert weights: blocks of 32 e2m1 values sharing one e8m0 scale (the
# 4-bit member of the same family: FlashInfer PR #3980 pairs its MXFP8 backend
# with 4-bit NVFP4 weights, and DeepGEMM PR #394 streams FP4 weight packets).
#
# Readings: e2m1 is the OCP FP4 encoding -- sign, 2 exponent bits with bias 1,
# 1 mantissa bit; exponent field 0 holds the subnormal m/2; no infinities or
# NaN; the values are 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Two codes per byte, the
# even-indexed value of a pair in the low nibble.  The block scale follows the
# OCP MX recipe with e2m1's top-binade exponent 2: 2^(floor(log2(amax)) - 2),
# code clamped to [0, 254], 0 for an all-zero block; elements are v / scale
# rounded to the nearest e2m1 value, ties to even mantissa, magnitudes above 6
# saturated to 6; the sign bit is the input's.
# ---------------------------------------------------------------------------
E2M1_MAX = 6.0


def _e2m1_value(c: np.ndarray) -> np.ndarray:
    """The E2M1 encoding written out: sign, exponent field, mantissa field."""
    c = c.astype(np.int64)
    sign = (c >> 3) & 1
    ex = (c >> 1) & 3
    man = c & 1
    mag = np.where(ex == 0, man * 0.5, (1.0 + man / 2.0) * np.exp2(ex - 1.0))
    return np.where(sign == 1, -mag, mag)


_E2M1_VALUES = _e2m1_value(np.arange(16))


def e2m1_to_f64(codes) -> np.ndarray:
    """Value of 4-bit E2M1 codes (0..15, one per array element) as float64."""
    return _E2M1_VALUES[np.asarray(codes, dtype=np.uint8) & 15]


def _round_to_e2m1(y: np.ndarray) -> np.ndarray:
    """Nearest e2m1 magnitude to |y|, ties to even mantissa, saturated at 6.
    Binade [2^E, 2^(E+1)), E >= 0, holds 2 values spaced 2^(E-1); below 1 the
    spacing is the subnormal step 1/2."""
    a = np.abs(y)
    _, ex = np.frexp(a)
    binade = np.maximum(ex - 1, 0)
    step = np.exp2(binade - 1.0)
    q = np.round(a / step) * step
    return np.minimum(q, E2M1_MAX)


def _encode_e2m1(mag: np.ndarray, sign: np.ndarray) -> np.ndarray:
    """Code (0..15) of an exactly representable e2m1 magnitude and a sign."""
    code = np.zeros(mag.shape, dtype=np.int64)
    sub = mag < 1.0
    code[sub] = np.rint(mag[sub] * 2.0).astype(np.int64)              # 0 or 1: field 0
    f, ex = np.frexp(mag[~sub])
    code[~sub] = (((ex - 1) + 1) << 1) | np.rint((f * 2.0 - 1.0) * 2.0).astype(np.int64)
    return code | (sign.astype(np.int64) << 3)


def mxfp4_quantize(w_bits):
    """MXFP4 quantization of bf16 weights along their last axis.

    w_bits: bf16 bits (uint16) [..., K], K a multiple of 32.  Returns
    (packed uint8 [..., K // 2], scales uint8 [..., K // 32]): byte i of a row
    holds the codes of values 2i (low nibble) and 2i + 1 (high nibble)."""
    b = np.ascontiguousarray(w_bits, dtype=np.uint16)
    K = b.shape[-1]
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    v = bf16_to_f64(b).reshape(b.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    amax = np.abs(v).max(axis=-1)
    _, ex = np.frexp(amax)
    s_code = np.where(amax > 0, np.clip((ex - 1) - 2 + 127, 0, 254), 0).astype(np.int64)
    y = v / np.exp2(s_code - 127.0)[..., None]
    mag = _round_to_e2m1(y)
    sign = (b.reshape(v.shape) >> np.uint16(15)).astype(np.int64)
    codes = _encode_e2m1(mag, sign).reshape(b.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, s_code.astype(np.uint8)


def mxfp4_to_f64(packed, scales) -> np.ndarray:
    """Dequantized MXFP4 weights [..., K]: e2m1 value times its block's scale."""
    p = np.asarray(packed, dtype=np.uint8)
    codes = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    codes[..., 0::2] = p & 15
    codes[..., 1::2] = p >> 4
    s = np.asarray(scales, dtype=np.uint8)
    return e2m1_to_f64(codes) * np.repeat(e8m0_to_f64(s), MX_BLOCK, axis=-1)


def forward_tokens_mxfp4(x, topk_ids, topk_weights, wgu_packed, wgu_scales, wd_packed, wd_scales,
                         tokens, num_valid_tokens: int | None = None, workers: int = 1):
    """forward_tokens with MXFP4 expert weights (packed codes [E, 2I, H/2] /
    scales [E, 2I, H/32], packed codes [E, H, I/2] / scales [E, H, I/32]),
    dequantized exactly to float64, then the same layer definition."""
    return forward_tokens_widened(
        x, topk_ids, topk_weights, len(wgu_packed),
        lambda e: (mxfp4_to_f64(wgu_packed[e], wgu_scales[e]), mxfp4_to_f64(wd_packed[e], wd_scales[e])),
        tokens, num_valid_tokens, workers)


def forward_mxfp4(x, topk_ids, topk_weights, wgu_packed, wgu_scales, wd_packed, wd_scales,
                  num_valid_tokens: int | None = None, workers: int = 1):
    """The whole MXFP4-weight layer for every token: float64 [T, H]."""
    T = np.asarray(topk_ids).shape[0]
    return forward_tokens_mxfp4(x, topk_ids, topk_weights, wgu_packed, wgu_scales, wd_packed,
                                wd_scales, np.arange(T), num_valid_tokens, workers)
