/*
 * moe_mi355x.h -- C ABI of the routed-MoE expert path for one AMD Instinct
 * MI355X (gfx950).  Exported by libmoe_mi355x.so.
 *
 * The layer computes, for every valid token t (t < T_v):
 *
 *   out[t,:] = sum_{j : 0 <= ids[t,j] < E}  w[t,j] * W_down[e] ( silu(W_gate[e] x[t]) * (W_up[e] x[t]) ),
 *   e = ids[t,j],  W_gate[e] = W_gateup[e, 0:I, :],  W_up[e] = W_gateup[e, I:2I, :],
 *
 * as the composition local dispatch -> dispatched-expert compute -> combine
 * (TileOps PR #1738 "[Refactor][MoE] Separate dispatched expert compute",
 * Summary), with the routing weights applied only in the combine (same
 * Summary), one (tokens, hidden) output (FlashInfer PR #3980, commit notes
 * on the kernel API migration, launch/output), a
 * tight no-pad expert-major batch whose expert_offsets stay on the GPU and
 * end in the valid-row count (TileOps PR #1738, Scope), and a static capacity
 * whose tail rows are unspecified (same Scope).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - bf16 tensors are passed as uint16_t bit patterns; all tensors are dense
 *    row-major, device memory, caller-owned.  bf16 pointers and the workspace
 *    must be 16-byte aligned, int32/fp32 pointers 4-byte aligned.  A pointer
 *    to an empty tensor (T = 0, or capacity 0) may be NULL.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Every call
 *    only enqueues work on it: no host synchronisation, no device-to-host
 *    read, no allocation, no memset.  All calls are therefore safe to record
 *    into a HIP graph.
 *  - Assignment a = t*K + j is valid iff t < T_v and 0 <= topk_ids[a] < E.
 *    Ids outside [0, E) (for example experts owned by another rank) are
 *    dropped, not errors.  T_v = T, or min(max(*num_tokens_dev, 0), T) when
 *    num_tokens_dev (a device int32) is given; it is read on the GPU.
 *  - Dispatched rows of one expert are ordered by increasing a (stable).
 *    Rows [R, capacity) of every dispatched buffer, and output rows t >= T_v,
 *    are left unspecified / untouched.
 *  - Arguments are checked on the host before anything is enqueued; a bad
 *    argument returns MOE_ERROR_INVALID_VALUE or MOE_ERROR_NOT_SUPPORTED and
 *    enqueues nothing (fail closed).  A failed launch returns
 *    MOE_ERROR_LAUNCH.  No entry point aborts or throws.
 *  - Arithmetic: bf16 inputs, fp32 accumulation, one round-to-nearest-even to
 *    bf16 for each of h, y and out.  No floating-point atomics: results are
 *    bit-reproducible run to run for a fixed problem and kernel plan.
 *  - A workspace must not be used by two calls that may run concurrently.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_problem {
    int32_t num_tokens;    /* T >= 0: rows of x and out (buffer rows)                  */
    int32_t top_k;         /* K, 1..64                                                 */
    int32_t num_experts;   /* E, 1..512: local experts (leading dim of the weights)    */
    int32_t hidden;        /* H > 0, multiple of 64                                    */
    int32_t intermediate;  /* I > 0, multiple of 64                                    */
    int32_t capacity;      /* rows of the dispatched buffers; 0 => T*K; must be >= T*K */
    int32_t kernel_hint;   /* grouped-GEMM plan: 0 auto (chosen from T*K/E on the host),
                              1 skinny (16-row tiles, in-workgroup split-K),
                              2 tiled 64-row, 3 tiled 128-row, 4 tiled large (192-row
                              tiles; 256-row when I is not a multiple of 128)         */
} moe_problem_t;

typedef enum moe_status {
    MOE_SUCCESS = 0,
    MOE_ERROR_INVALID_VALUE = 1,
    MOE_ERROR_NOT_SUPPORTED = 2,
    MOE_ERROR_LAUNCH = 3
} moe_status_t;

/* Human-readable text of a status (static storage).  The statuses are those
 * of the host-side validation that rejects unsupported shapes before any work
 * is enqueued (DeepGEMM PR #394, Scope and fallback: unsupported shapes fail
 * closed during host validation). */
MOE_API const char* moe_status_string(moe_status_t status);

/* Bytes of device workspace every entry point below needs for `p` (the
 * largest of them, moe_forward).  Host-only.  Returns MOE_ERROR_* for an
 * invalid problem and leaves *bytes untouched.  The workspace is a
 * caller-owned buffer passed into each call (TileOps PR #1738, Scope: buffers
 * injected by the caller; FlashInfer PR #3980, commit notes on the workspace
 * contract: a workspace is set up once and every launch leaves it ready for
 * the next).  Unlike the counters of that contract, nothing in this
 * workspace needs initialising or cleaning: each call writes every region it
 * reads before reading it. */
MOE_API moe_status_t moe_workspace_size(const moe_problem_t* p, size_t* bytes);

/* Local dispatch (TileOps PR #1738, Summary: local dispatch into a tight
 * expert-major batch; Scope: GPU-resident expert_offsets[-1:] valid-row view).
 *   x               bf16 [T, H]
 *   topk_ids        int32 [T, K]
 *   num_tokens_dev  device int32 scalar or NULL (see T_v above)
 *   x_disp          out bf16 [capacity, H]: row r = x[row_src[r] / K]
 *   expert_offsets  out int32 [E+1]: exclusive prefix of per-expert counts;
 *                   expert_offsets[E] = R, the valid-row count
 *   row_src         out int32 [capacity]: assignment a of row r (r < R)
 *   token_row       out int32 [T*K]: row of assignment a, -1 if dropped
 *   workspace       >= moe_workspace_size bytes (ws_bytes is checked)
 * Results are exact integers / bit copies. */
MOE_API moe_status_t moe_dispatch(const moe_problem_t* p, const uint16_t* x, const int32_t* topk_ids,
                          const int32_t* num_tokens_dev, uint16_t* x_disp,
                          int32_t* expert_offsets, int32_t* row_src, int32_t* token_row,
                          void* workspace, size_t ws_bytes, void* stream);

/* Dispatched-expert compute over a tight expert-major batch (TileOps PR
 * #1738, Summary and Review follow-up: gate-up grouped GEMM, fused gated
 * pointwise epilogue, down grouped GEMM).  Routing weights are not inputs.
 *   x_disp          bf16 [capacity, H]; rows [0, R) are read
 *   expert_offsets  int32 [E+1] on the device (as written by moe_dispatch)
 *   w_gateup        bf16 [E, 2I, H]: rows [0, I) gate, rows [I, 2I) up
 *   w_down          bf16 [E, H, I]
 *   y_disp          out bf16 [capacity, H]: rows [0, R) written
 *   workspace       holds h = bf16(silu(gate) * up) [capacity, I] */
MOE_API moe_status_t moe_expert_compute(const moe_problem_t* p, const uint16_t* x_disp,
                                const int32_t* expert_offsets, const uint16_t* w_gateup,
                                const uint16_t* w_down, uint16_t* y_disp,
                                void* workspace, size_t ws_bytes, void* stream);

/* The two grouped GEMMs of moe_expert_compute as separate calls (TileOps PR
 * #1738, Review follow-up: gate-up and down grouped-GEMM sub-ops), for
 * callers that schedule or time them individually.
 *   moe_gate_up: h [capacity, I] = bf16( silu(x_disp W_gate[e]^T) * (x_disp W_up[e]^T) )
 *   moe_down:    y_disp [capacity, H] = bf16( h W_down[e]^T )
 * for every dispatched row r < R of expert e (expert_offsets[e] <= r <
 * expert_offsets[e+1]), fp32 accumulation.  Same kernels and plan as
 * moe_expert_compute, so the pair reproduces it bit for bit. */
MOE_API moe_status_t moe_gate_up(const moe_problem_t* p, const uint16_t* x_disp,
                                 const int32_t* expert_offsets, const uint16_t* w_gateup,
                                 uint16_t* h, void* stream);
MOE_API moe_status_t moe_down(const moe_problem_t* p, const uint16_t* h,
                              const int32_t* expert_offsets, const uint16_t* w_down,
                              uint16_t* y_disp, void* stream);

/* Weighted top-k combine back to token order (TileOps PR #1738, Summary:
 * weights stay outside expert compute; FlashInfer PR #3980, kernel API
 * migration notes: one (tokens, hidden) output).  For t < T_v:
 *   out[t,:] = bf16( sum_{j ascending, token_row[t*K+j] >= 0} w[t,j] * y_disp[token_row[t*K+j], :] )
 * accumulated in fp32 (a zero row when no assignment is valid).
 *   y_disp bf16 [capacity, H], token_row int32 [T*K], topk_weights fp32 [T, K],
 *   out bf16 [T, H] (rows t >= T_v untouched). */
MOE_API moe_status_t moe_combine(const moe_problem_t* p, const uint16_t* y_disp, const int32_t* token_row,
                         const float* topk_weights, const int32_t* num_tokens_dev,
                         uint16_t* out, void* stream);

/* Router top-k, the step ahead of moe_dispatch (TileOps PR #1738, Summary:
 * routing weights are produced outside expert compute).  For t < T_v and the
 * E = num_experts router logits of token t:
 *   topk_ids[t, 0..K-1]     indices of the K largest logits, in decreasing
 *                           order; equal values in increasing index
 *   topk_weights[t, j]      exp(l_j - l_0) / sum_{i<K} exp(l_i - l_0) over the
 *                           selected logits l_0 >= l_1 >= ... (fp32, sum in
 *                           increasing j)
 *   logits fp32 [T, E] (finite values; -0 and +0 are equal), topk_ids int32
 *   [T, K], topk_weights fp32 [T, K]; rows t >= T_v are not written.
 * Requires K <= E.  The outputs feed moe_dispatch / moe_forward directly.
 * hidden, intermediate and capacity are not used beyond the usual checks. */
MOE_API moe_status_t moe_router_topk(const moe_problem_t* p, const float* logits,
                                     const int32_t* num_tokens_dev, int32_t* topk_ids,
                                     float* topk_weights, void* stream);

/* The router step fused ahead of dispatch: the dispatch kernels take each
 * token's top-K of its router logits themselves, with no launch of their own
 * (TileOps PR #1738, Summary: the routing weights are produced outside expert
 * compute and carried beside the ids).  For t < T_v and the G = router_experts
 * logits of token t (fp32 [T, G], finite; -0 equal to +0):
 *   topk_ids[t, 0..K-1]   out: indices of the K largest logits, decreasing,
 *                         equal values in increasing index (global ids: only
 *                         those below num_experts are local, the rest are
 *                         dropped by the dispatch like any non-local id)
 *   topk_weights[t, j]    out: exp(l_j - l_0) / sum_{i<K} exp(l_i - l_0) over
 *                         the selected logits, fp32, summed in increasing j
 * (the ids and weights moe_router_topk gives with num_experts = G, bit for
 * bit), then moe_dispatch on those ids: x_disp, expert_offsets, row_src,
 * token_row as there.  Rows t >= T_v of topk_ids / topk_weights are not
 * written.  Requires 1 <= K <= G <= 65536 (MOE_ERROR_INVALID_VALUE /
 * MOE_ERROR_NOT_SUPPORTED otherwise).  topk_ids int32 [T, K], topk_weights
 * fp32 [T, K], logits 4-byte aligned. */
MOE_API moe_status_t moe_router_dispatch(const moe_problem_t* p, int32_t router_experts,
                                         const float* logits, const int32_t* num_tokens_dev,
                                         int32_t* topk_ids, float* topk_weights,
                                         const uint16_t* x, uint16_t* x_disp,
                                         int32_t* expert_offsets, int32_t* row_src,
                                         int32_t* token_row, void* workspace, size_t ws_bytes,
                                         void* stream);

/* The whole layer from router logits: the router step fused into the dispatch
 * (as in moe_router_dispatch; topk_ids / topk_weights are written), then
 * expert compute and combine.  Equal bit for bit to moe_router_topk (with
 * num_experts = router_experts) followed by moe_forward on its outputs. */
MOE_API moe_status_t moe_forward_logits(const moe_problem_t* p, int32_t router_experts,
                                        const float* logits, const uint16_t* x,
                                        const uint16_t* w_gateup, const uint16_t* w_down,
                                        const int32_t* num_tokens_dev, int32_t* topk_ids,
                                        float* topk_weights, int32_t* expert_offsets,
                                        uint16_t* out, void* workspace, size_t ws_bytes,
                                        void* stream);

/* The whole layer: dispatch, expert compute (the row gather fused into the
 * gate-up GEMM's operand loads) and combine, enqueued back to back.
 *   expert_offsets  out int32 [E+1] (the GPU-resident valid-row view)
 *   out             bf16 [T, H]
 * Equal bit for bit to moe_dispatch + moe_expert_compute + moe_combine with
 * the same kernel plan. */
MOE_API moe_status_t moe_forward(const moe_problem_t* p, const uint16_t* x, const int32_t* topk_ids,
                         const float* topk_weights, const uint16_t* w_gateup,
                         const uint16_t* w_down, const int32_t* num_tokens_dev,
                         int32_t* expert_offsets, uint16_t* out,
                         void* workspace, size_t ws_bytes, void* stream);

/* The whole layer in ONE launch, for tiny batches (TileOps PR #1738, review
 * comments: one megakernel for dispatch, expert compute and combine;
 * FlashInfer PR #3980, kernel API migration notes: the top-k combine reduced
 * inside the kernel).  Same arguments, checks and result as moe_forward, bit
 * for bit.  Serves T*K <= 8 with I % 1024 == 0 and kernel_hint 0 or 1 (the
 * latency-bound decode regime, where a launch is a large part of the layer);
 * other problems return MOE_ERROR_NOT_SUPPORTED, as does a device that cannot
 * hold the launch's grid at once.  The launch is cooperative: a persistent
 * grid runs the dispatch and the gate-up tiles, waits at a grid-wide barrier,
 * then runs the down GEMM and the combine.  The barrier lives in one
 * library-owned device variable per GPU; its wait is bounded: past about 0.3 s
 * it records a timeout (read with moe_single_launch_status) and the launch
 * finishes with undefined output rather than hanging.  Launches of it on one
 * GPU must not overlap (they cannot share the device anyway: each takes all of
 * it).  Not for graph capture (a cooperative launch). */
MOE_API moe_status_t moe_forward_single(const moe_problem_t* p, const uint16_t* x,
                                        const int32_t* topk_ids, const float* topk_weights,
                                        const uint16_t* w_gateup, const uint16_t* w_down,
                                        const int32_t* num_tokens_dev, int32_t* expert_offsets,
                                        uint16_t* out, void* workspace, size_t ws_bytes,
                                        void* stream);

/* Barrier timeouts recorded by moe_forward_single on the current device since
 * the last call (0 when every launch completed normally), then resets the
 * barrier state.  Host-synchronous: call it with no moe_forward_single in
 * flight on the device. */
MOE_API moe_status_t moe_single_launch_status(uint32_t* barrier_timeouts);

/* Static-capacity graph replay (TileOps PR #1738, Summary: GPU-resident row
 * counts, static capacity and graph replay).  Records one moe_forward with
 * these fixed pointers into an instantiated HIP graph; every launch in it has
 * a fixed grid and reads T_v and all row counts on the GPU, so the caller
 * replays it after writing new x / topk_ids / topk_weights / *num_tokens_dev
 * into the same buffers.  *graph_out receives an opaque handle owned by the
 * caller (release with moe_graph_destroy). */
MOE_API moe_status_t moe_graph_create(const moe_problem_t* p, const uint16_t* x, const int32_t* topk_ids,
                              const float* topk_weights, const uint16_t* w_gateup,
                              const uint16_t* w_down, const int32_t* num_tokens_dev,
                              int32_t* expert_offsets, uint16_t* out,
                              void* workspace, size_t ws_bytes, void** graph_out);
MOE_API moe_status_t moe_graph_launch(void* graph, void* stream);
MOE_API moe_status_t moe_graph_destroy(void* graph);

/* moe_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The
 * same layer, kernels, plan, checks and results (bit for bit) as moe_forward,
 * with the workspace taken from a library-owned file-scope device array of
 * 128 MiB instead of a caller buffer; each GPU holds its own copy of that
 * array from the library's first call there until the process ends.
 *  - Problems whose moe_forward workspace (moe_workspace_size) exceeds 128 MiB
 *    return MOE_ERROR_NOT_SUPPORTED, checked on the host before anything
 *    else happens (for example the 96-expert decode shares up to T = 128 and
 *    the static-capacity layer of 16384 rows fit; a 4096-token Mixtral-style
 *    layer does not).
 *  - It calls no hipMalloc / hipFree and no allocating routine.  The first call
 *    on a device looks up the array's address there (hipGetSymbolAddress, with
 *    the calling thread's current device, which must be the device of
 *    `stream`); make that first call outside a graph capture.
 *  - Every call on one GPU shares that GPU's array, whose contents are left
 *    from the last call (nothing in it needs clearing: each region is written
 *    before it is read).  Calls that may overlap on one GPU (concurrent
 *    streams, or a replayed graph holding this call racing an eager one) race
 *    on it and must be serialised by the caller.
 * Arguments as for moe_forward without workspace / ws_bytes. */
MOE_API moe_status_t moe_forward_noalloc(const moe_problem_t* p, const uint16_t* x,
                                         const int32_t* topk_ids, const float* topk_weights,
                                         const uint16_t* w_gateup, const uint16_t* w_down,
                                         const int32_t* num_tokens_dev, int32_t* expert_offsets,
                                         uint16_t* out, void* stream);

/* ---------------------------------------------------------------------------
 * Pre-packed bf16 expert weights for the weight-streaming (skinny) kernels
 * (DeepGEMM PR #394, Summary and Motivation: expert weights laid out once, at
 * load, in the order the kernel reads them, the row-major layout staying the
 * reference; Correctness: the packed path checked bit for bit against it).
 *
 * moe_skinny_pack rewrites w [experts, rows, k] (bf16, row-major; k % 32 == 0,
 * rows % 16 == 0) into packed [experts, rows, k] of the same size: 16-row
 * groups, each stored as [k/32 steps][64 lanes][8 values], lane l holding row
 * l%16 of the group and k-values 32s + 8(l/16) .. +7 of step s.  Plain
 * (gated = 0, for W_down [E, H, I]): group g = rows 16g .. 16g+15.  Gated
 * (gated = 1, for W_gateup [E, 2I, H]): group g = gate rows 8g .. 8g+7 and the
 * matching up rows I+8g .. I+8g+7.  w and packed must not overlap; both
 * 16-byte aligned.  experts * rows * k <= 2^40. */
MOE_API moe_status_t moe_skinny_pack(const uint16_t* w, int32_t experts, int32_t rows, int32_t k,
                                     int32_t gated, uint16_t* packed, void* stream);

/* moe_gate_up / moe_forward on packed weights (W_gateup packed gated, W_down
 * packed plain).  They run the skinny plan for every batch size (kernel_hint
 * 0 or 1; MOE_ERROR_NOT_SUPPORTED otherwise) and are bit-identical to
 * moe_gate_up / moe_forward with kernel_hint = 1 on the row-major weights. */
MOE_API moe_status_t moe_gate_up_packed(const moe_problem_t* p, const uint16_t* x_disp,
                                        const int32_t* expert_offsets,
                                        const uint16_t* w_gateup_packed, uint16_t* h,
                                        void* stream);
MOE_API moe_status_t moe_forward_packed(const moe_problem_t* p, const uint16_t* x,
                                        const int32_t* topk_ids, const float* topk_weights,
                                        const uint16_t* w_gateup_packed,
                                        const uint16_t* w_down_packed,
                                        const int32_t* num_tokens_dev, int32_t* expert_offsets,
                                        uint16_t* out, void* workspace, size_t ws_bytes,
                                        void* stream);

/* ---------------------------------------------------------------------------
 * Pre-packed bf16 expert weights for the tiled (prefill) kernels (DeepGEMM PR
 * #394, Summary and Motivation: weights laid out once in the kernel's access
 * order; Correctness: checked bit for bit against the row-major path).
 *
 * moe_tiled_pack rewrites w [experts, rows, k] (bf16; rows % 32 == 0, k % 64
 * == 0) into packed of the same size: for expert e, 8-row group g and stage s
 * (k-values 64s .. 64s+63) one contiguous 1 KiB block of 64 pieces of 8
 * values, piece L = row 8g + L/8, k-values 64s + 8c .. +7 with
 * c = (L % 8) ^ swz((8g + L/8) % 32), swz(r) = ((r >> 1) & 3) | ((r >> 2) & 4):
 * exactly the 1 KiB one DMA instruction of the tiled kernels stages, in LDS
 * slot order.  Both W_gateup [E, 2I, H] and W_down [E, H, I] are packed the
 * same way.  w and packed must not overlap; both 16-byte aligned.
 * ------------------------------------------------------------------------- */
MOE_API moe_status_t moe_tiled_pack(const uint16_t* w, int32_t experts, int32_t rows, int32_t k,
                                    uint16_t* packed, void* stream);

/* moe_gate_up / moe_forward on weights packed by moe_tiled_pack.  They run a
 * tiled plan (kernel_hint 2, 3, 4, or 0: the automatic choice, with the
 * 64-row tiled plan where it would pick the skinny one; kernel_hint 1 returns
 * MOE_ERROR_NOT_SUPPORTED) and are bit-identical to moe_gate_up / moe_forward
 * with that plan on the row-major weights. */
MOE_API moe_status_t moe_gate_up_tiled_packed(const moe_problem_t* p, const uint16_t* x_disp,
                                              const int32_t* expert_offsets,
                                              const uint16_t* w_gateup_packed, uint16_t* h,
                                              void* stream);
MOE_API moe_status_t moe_forward_tiled_packed(const moe_problem_t* p, const uint16_t* x,
                                              const int32_t* topk_ids, const float* topk_weights,
                                              const uint16_t* w_gateup_packed,
                                              const uint16_t* w_down_packed,
                                              const int32_t* num_tokens_dev,
                                              int32_t* expert_offsets, uint16_t* out,
                                              void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * MXFP8 expert weights (FlashInfer PR #3980: the MXFP8 MegaMoE backend; its
 * combine-wire notes name the format, 32 e4m3 values sharing one e8m0 scale).
 * TileOps PR #1738, Scope, leaves FP8 outside its BF16 path; this is the
 * low-precision weight variant of the same layer, for the weight-streaming
 * regime: about half the weight bytes of bf16.
 *
 * Format of a weight matrix with K-contiguous rows [rows, K], K % 32 == 0:
 *   codes   uint8 [rows, K]: OCP FP8 E4M3 ("fn": bias 7, subnormals, no
 *           infinities, 0x7F / 0xFF NaN, largest value 448)
 *   scales  uint8 [rows, K/32]: e8m0, code s means 2^(s - 127), one per 32
 *           consecutive values of a row
 *   value(r, k) = e4m3(codes[r, k]) * 2^(scales[r, k/32] - 127)
 * For the layer: W_gateup codes [E, 2I, H] + scales [E, 2I, H/32] (gate rows
 * first), W_down codes [E, H, I] + scales [E, H, I/32].  codes 16-byte
 * aligned, scales 2-byte aligned.
 * ------------------------------------------------------------------------- */

/* Quantize bf16 rows w [rows, k] (16-byte aligned) to MXFP8: per block of 32
 * the scale is 2^(floor(log2(amax)) - 8), its code clamped to [0, 254] (0 for
 * an all-zero block); each code is the nearest e4m3 value to v / scale, ties
 * to even, magnitudes above 448 saturated to 448, sign bit = the input's.
 * Exact integer arithmetic (the result is bit-reproducible).  Finite inputs
 * only.  rows >= 0, k a positive multiple of 32; rows * k <= 2^40. */
MOE_API moe_status_t moe_mxfp8_quantize(const uint16_t* w, int64_t rows, int32_t k,
                                        uint8_t* codes, uint8_t* scales, void* stream);

/* Dequantize MXFP8 rows to bf16 w [rows, k] with the conversion the expert
 * kernels use (v_cvt_scalef32_pk_bf16_fp8).  Exact for scale codes whose
 * results stay in bf16's normal range (every code the quantizer gives for
 * weights between 2^-117 and 2^119 in magnitude). */
MOE_API moe_status_t moe_mxfp8_dequantize(const uint8_t* codes, const uint8_t* scales,
                                          int64_t rows, int32_t k, uint16_t* w, void* stream);

/* moe_gate_up on MXFP8 gate-up weights: h = bf16(silu(x_disp W_gate^T) *
 * (x_disp W_up^T)) with the weights dequantized exactly in registers and fp32
 * accumulation.  kernel_hint must be 0 or 1 (the 16-row skinny tiles serve
 * every batch size on this path); MOE_ERROR_NOT_SUPPORTED otherwise. */
MOE_API moe_status_t moe_gate_up_mxfp8(const moe_problem_t* p, const uint16_t* x_disp,
                                       const int32_t* expert_offsets,
                                       const uint8_t* w_gateup_codes,
                                       const uint8_t* w_gateup_scales, uint16_t* h,
                                       void* stream);

/* moe_forward on MXFP8 expert weights: the same layer, dispatch, combine,
 * workspace, T_v handling and output contract, with W_gateup and W_down given
 * as codes + scales (above).  x, h, y and out stay bf16.  kernel_hint 0 or 1. */
MOE_API moe_status_t moe_forward_mxfp8(const moe_problem_t* p, const uint16_t* x,
                                       const int32_t* topk_ids, const float* topk_weights,
                                       const uint8_t* w_gateup_codes,
                                       const uint8_t* w_gateup_scales,
                                       const uint8_t* w_down_codes,
                                       const uint8_t* w_down_scales,
                                       const int32_t* num_tokens_dev, int32_t* expert_offsets,
                                       uint16_t* out, void* workspace, size_t ws_bytes,
                                       void* stream);

/* ---------------------------------------------------------------------------
 * MXFP4 expert weights: the 4-bit member of the same family (FlashInfer PR
 * #3980 pairs its MXFP8 backend with 4-bit NVFP4 weights; DeepGEMM PR #394,
 * Summary, streams FP4 expert weights), a quarter of the bf16 weight bytes.
 *
 * Format of a weight matrix with K-contiguous rows [rows, K], K % 32 == 0:
 *   codes   uint8 [rows, K/2]: OCP FP4 E2M1 codes (sign, 2 exponent bits with
 *           bias 1, 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities
 *           or NaN), two per byte, value 2i in the low nibble of byte i
 *   scales  uint8 [rows, K/32]: e8m0, one per 32 consecutive values of a row
 *   value(r, k) = e2m1(code(r, k)) * 2^(scales[r, k/32] - 127)
 * For the layer: W_gateup codes [E, 2I, H/2] + scales [E, 2I, H/32], W_down
 * codes [E, H, I/2] + scales [E, H, I/32].  codes 16-byte aligned, scales
 * 4-byte aligned; H and I multiples of 128 (MOE_ERROR_NOT_SUPPORTED
 * otherwise).
 * ------------------------------------------------------------------------- */

/* Quantize bf16 rows w [rows, k] to MXFP4: per block of 32 the scale is
 * 2^(floor(log2(amax)) - 2), its code clamped to [0, 254] (0 for an all-zero
 * block); each code is the nearest e2m1 value to v / scale, ties to even,
 * magnitudes above 6 saturated to 6, sign bit = the input's.  Exact integer
 * arithmetic.  Same argument rules as moe_mxfp8_quantize. */
MOE_API moe_status_t moe_mxfp4_quantize(const uint16_t* w, int64_t rows, int32_t k,
                                        uint8_t* codes, uint8_t* scales, void* stream);

/* Dequantize MXFP4 rows to bf16 w [rows, k] with the conversion the expert
 * kernels use (v_cvt_scalef32_pk_bf16_fp4); exact whenever the result is a
 * normal bf16 value. */
MOE_API moe_status_t moe_mxfp4_dequantize(const uint8_t* codes, const uint8_t* scales,
                                          int64_t rows, int32_t k, uint16_t* w, void* stream);

/* moe_gate_up_mxfp8 / moe_forward_mxfp8 with MXFP4 weights (same contracts). */
MOE_API moe_status_t moe_gate_up_mxfp4(const moe_problem_t* p, const uint16_t* x_disp,
                                       const int32_t* expert_offsets,
                                       const uint8_t* w_gateup_codes,
                                       const uint8_t* w_gateup_scales, uint16_t* h,
                                       void* stream);
MOE_API moe_status_t moe_forward_mxfp4(const moe_problem_t* p, const uint16_t* x,
                                       const int32_t* topk_ids, const float* topk_weights,
                                       const uint8_t* w_gateup_codes,
                                       const uint8_t* w_gateup_scales,
                                       const uint8_t* w_down_codes,
                                       const uint8_t* w_down_scales,
                                       const int32_t* num_tokens_dev, int32_t* expert_offsets,
                                       uint16_t* out, void* workspace, size_t ws_bytes,
                                       void* stream);

/* ---------------------------------------------------------------------------
 * MX codes in the skinny pack layout (the layout of moe_skinny_pack, on the
 * code bytes): the MX decode kernels then read each wave's codes as one
 * contiguous run.  Measured 7-17% faster than row-major codes on the decode
 * workloads; the scales stay row-major.
 * ------------------------------------------------------------------------- */

/* Pack MX codes [experts, rows, k * bits / 8 bytes] (bits = 8: MXFP8, 4:
 * MXFP4; k values per row) into the skinny pack layout: moe_skinny_pack on
 * the codes viewed as 16-bit values with k' = k * bits / 16 per row (so k *
 * bits must be a multiple of 512, rows a multiple of 16).  gated = 1 for the
 * W_gateup codes, 0 for W_down.  Same size; no overlap; 16-byte aligned. */
MOE_API moe_status_t moe_mx_pack(const uint8_t* codes, int32_t experts, int32_t rows, int32_t k,
                                 int32_t bits, int32_t gated, uint8_t* packed, void* stream);

/* moe_gate_up_mxfp8 / _mxfp4 and moe_forward_mxfp8 / _mxfp4 (bits = 8 / 4) on
 * codes packed by moe_mx_pack, with the same row-major scales; bit-identical
 * to the row-major entry points. */
MOE_API moe_status_t moe_gate_up_mx_packed(const moe_problem_t* p, int32_t bits,
                                           const uint16_t* x_disp, const int32_t* expert_offsets,
                                           const uint8_t* w_gateup_codes_packed,
                                           const uint8_t* w_gateup_scales, uint16_t* h,
                                           void* stream);
MOE_API moe_status_t moe_forward_mx_packed(const moe_problem_t* p, int32_t bits, const uint16_t* x,
                                           const int32_t* topk_ids, const float* topk_weights,
                                           const uint8_t* w_gateup_codes_packed,
                                           const uint8_t* w_gateup_scales,
                                           const uint8_t* w_down_codes_packed,
                                           const uint8_t* w_down_scales,
                                           const int32_t* num_tokens_dev, int32_t* expert_offsets,
                                           uint16_t* out, void* workspace, size_t ws_bytes,
                                           void* stream);

/* ---------------------------------------------------------------------------
 * MX codes in the tiled pack layout, for the tiled (prefill) kernels on MX
 * weights (DeepGEMM PR #394, Summary and Motivation: weights laid out once in
 * the kernel's access order; FlashInfer PR #3980, Summary: the MXFP8
 * backend).  The tiled MX kernels stage a weight tile's codes as 1 KiB DMA
 * pieces of 16 rows x 64 bytes (e4m3: 64 values of a row per stage) or 32
 * rows x 32 bytes (e2m1), row r's 16-byte chunk c in LDS slot c ^ swz(r % 32)
 * with swz8(r) = ((r >> 2) & 1) | ((r >> 3) & 2) and swz4(r) = (r >> 4) & 1.
 * Row-major, each piece gathers 16 or 32 partial cache lines; packed, it is
 * one contiguous 1 KiB.
 *
 * moe_mx_tiled_pack rewrites codes [experts, rows, k * bits / 8 bytes] (bits =
 * 8: MXFP8, 4: MXFP4; k values per row; rows % 32 == 0, k % 64 == 0) into
 * packed of the same size: for expert e, group g of 1024 / (64 * bits / 8)
 * rows and stage s (values 64s .. 64s+63), one 1 KiB block whose 16-byte
 * piece L holds row g * G + L / C (G rows per group, C = 64 * bits / 128
 * chunks per row and stage), chunk (L % C) ^ swz(row % 32) of that row's
 * stage.  codes and packed must not overlap; both 16-byte aligned; the
 * scales stay row-major.  Both W_gateup [E, 2I, .] and W_down [E, H, .]
 * codes are packed the same way. */
MOE_API moe_status_t moe_mx_tiled_pack(const uint8_t* codes, int32_t experts, int32_t rows,
                                       int32_t k, int32_t bits, uint8_t* packed, void* stream);

/* moe_gate_up_mxfp8 / _mxfp4 and moe_forward_mxfp8 / _mxfp4 (bits = 8 / 4) on
 * codes packed by moe_mx_tiled_pack, with the same row-major scales.  They run
 * a tiled plan (kernel_hint 2, 3, 4, or 0: the automatic choice, with the
 * 64-row tiled plan where it would pick the skinny one; kernel_hint 1 returns
 * MOE_ERROR_NOT_SUPPORTED), need hidden (and, for the forward, intermediate)
 * a multiple of 512 and at most 7168 (the tile's scales fit in LDS), else
 * MOE_ERROR_NOT_SUPPORTED, and are bit-identical to the row-major entry
 * points with that plan. */
MOE_API moe_status_t moe_gate_up_mx_tiled_packed(const moe_problem_t* p, int32_t bits,
                                                 const uint16_t* x_disp,
                                                 const int32_t* expert_offsets,
                                                 const uint8_t* w_gateup_codes_tiled,
                                                 const uint8_t* w_gateup_scales, uint16_t* h,
                                                 void* stream);
MOE_API moe_status_t moe_forward_mx_tiled_packed(const moe_problem_t* p, int32_t bits,
                                                 const uint16_t* x, const int32_t* topk_ids,
                                                 const float* topk_weights,
                                                 const uint8_t* w_gateup_codes_tiled,
                                                 const uint8_t* w_gateup_scales,
                                                 const uint8_t* w_down_codes_tiled,
                                                 const uint8_t* w_down_scales,
                                                 const int32_t* num_tokens_dev,
                                                 int32_t* expert_offsets, uint16_t* out,
                                                 void* workspace, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
