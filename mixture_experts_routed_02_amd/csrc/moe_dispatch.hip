// Local dispatch of top-k routed assignments into a tight, unpadded,
// expert-major batch (TileOps PR #1738 "[Refactor][MoE] Separate dispatched
// expert compute", Summary and Scope): per-expert histogram, exclusive scan
// into expert_offsets (last entry = valid-row count, left on the GPU), and a
// stable scatter that keeps the rows of one expert in increasing assignment
// order a = t*K + j.
//
// Small problems (T*K <= kDispatchSingleMax) run as one 1024-thread block.
// Larger ones run a per-block histogram into the workspace, then the scatter,
// in which every block takes its own start inside each expert and the
// totals from those histograms (no atomics across blocks, nothing to reset
// between calls).  With many blocks, an exclusive scan of each expert's
// column over the blocks (one workgroup per expert; the column total goes to
// an extra row) runs in between, so the work stays linear in the number of
// blocks; with few, each scatter block sums the rows before its own.
// With the router fused ahead (router_* entry points), the same kernels first
// take each token's top-K of its router logits (route_token below) and use
// those ids; the counting kernel routes for the multi-block form and writes
// the ids for the scatter.
//
// Within a block, ranks among equal experts come from wave64 ballots: one
// ballot per bit of the expert id gives each lane the mask of lanes holding
// its expert, and the lane's rank is the popcount of that mask below it plus
// the count of that expert earlier in the wave's slice; per-wave counts are
// then scanned across waves in LDS.
#include "moe_internal.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// Router step fused ahead of dispatch (TileOps PR #1738, Summary: routing
// weights are produced outside expert compute and carried beside the ids).
// One lane per token: the K largest of its G logits in decreasing order,
// equal values in increasing index (-0 equal to +0), and the softmax over the
// selected values, w_j = exp(v_j - v_0) / sum_{i<K} exp(v_i - v_0), fp32, the
// sum in increasing j -- the arithmetic of router_topk_kernel, so both give
// the same ids and weights bit for bit.  Each pick is one pass over the row:
// the largest logit strictly after the previous pick in that order.  A first
// round of picks gives the sum, a second one emits (the picks and each
// exp are the same both times).  Finite logits assumed.
// ---------------------------------------------------------------------------
struct Pick {
    float v;
    int i;
};

// Rows of at most kRouteRegs logits are read into registers, kRouteBatch
// tokens per thread at a time with all their loads issued together (the
// routing of a single block is otherwise one memory round trip per token);
// longer rows are scanned in memory on every pick.
constexpr int kRouteRegs = 8;
constexpr int kRouteBatch = 4;

// The next pick after `prev` among register slots r[0..kRouteRegs) (slots
// past G hold -inf, which never beats a finite logit): straight-line selects.
__device__ __forceinline__ Pick next_pick_regs(const float* r, Pick prev) {
    float bv = -INFINITY;
    int bi = 0;
#pragma unroll
    for (int i = 0; i < kRouteRegs; ++i) {
        const float v = r[i];
        const bool take = (v < prev.v || (v == prev.v && i > prev.i)) && v > bv;
        bv = take ? v : bv;
        bi = take ? i : bi;
    }
    // -0 equals +0: report the value as +0, as the wave-wide router does
    return Pick{bv == 0.f ? 0.f : bv, bi};
}

// The same over a row of G logits in memory.
__device__ __forceinline__ Pick next_pick_mem(const float* __restrict__ row, int G, Pick prev) {
    float bv = -INFINITY;
    int bi = 0;
    for (int i = 0; i < G; ++i) {
        const float v = row[i];
        const bool take = (v < prev.v || (v == prev.v && i > prev.i)) && v > bv;
        bv = take ? v : bv;
        bi = take ? i : bi;
    }
    return Pick{bv == 0.f ? 0.f : bv, bi};
}

// emit(j, expert, weight) for the K picks of one token: with REGS its logits
// are r[0..kRouteRegs), else the row `row` of G logits.  K is the same for
// every lane, so the pick loops are scalar loops.
template <bool REGS, typename EMIT>
__device__ __forceinline__ void route_token(const float* __restrict__ row, const float* r, int G,
                                            int K, EMIT emit) {
    auto pick = [&](Pick prev) { return REGS ? next_pick_regs(r, prev) : next_pick_mem(row, G, prev); };
    Pick p{INFINITY, -1};
    float v0 = 0.f, sum = 0.f;
    for (int j = 0; j < K; ++j) {
        p = pick(p);
        if (j == 0) v0 = p.v;
        sum += expf(p.v - v0);
    }
    p = Pick{INFINITY, -1};
    for (int j = 0; j < K; ++j) {
        p = pick(p);
        emit(j, p.i, expf(p.v - v0) / sum);
    }
}

// Route the tokens that own assignments [a0, a1) (t < T_v only): s_ids[a -
// a0] = expert of assignment a; topk_ids / topk_weights written for the
// assignments in [a0, a1).  A token whose assignments straddle two blocks is
// routed by both, with the same result.  With REGS each thread loads the
// rows of kRouteBatch tokens together (unconditional loads of a clamped row,
// then -inf past G).  Ends with a barrier.
template <bool REGS>
__device__ __forceinline__ void route_block(const float* __restrict__ logits, int G, int K,
                                            int tv, long long a0, long long a1, int* s_ids,
                                            int32_t* __restrict__ ids_out,
                                            float* __restrict__ w_out) {
    const int t0 = (int)(a0 / K);
    const int t1 = (int)((a1 + K - 1) / K < tv ? (a1 + K - 1) / K : tv);
    constexpr int NB = REGS ? kRouteBatch : 1;
    const int nt = blockDim.x;
    for (int tb = t0 + (int)threadIdx.x; tb < t1; tb += NB * nt) {
        float r[NB][REGS ? kRouteRegs : 1];
        if (REGS) {
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const int t = tb + u * nt < t1 ? tb + u * nt : t1 - 1;
                const float* row = logits + (size_t)t * G;
#pragma unroll
                for (int i = 0; i < kRouteRegs; ++i) r[u][i] = row[i < G ? i : 0];
#pragma unroll
                for (int i = 0; i < kRouteRegs; ++i) r[u][i] = i < G ? r[u][i] : -INFINITY;
            }
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int t = tb + u * nt;
            if (t < t1)
                route_token<REGS>(logits + (size_t)t * G, r[u], G, K, [&](int j, int e, float w) {
                    const long long a = (long long)t * K + j;
                    if (a >= a0 && a < a1) {
                        s_ids[a - a0] = e;
                        ids_out[a] = e;
                        w_out[a] = w;
                    }
                });
        }
    }
    __syncthreads();
}

// Per-block histograms of CHUNK assignments each (block b: [b*CHUNK,
// (b+1)*CHUNK)) into row b of blk_counts.  ROUTE: the block first routes the
// tokens of its chunk (routing is what limits these blocks, so the routed
// form uses chunks of 1024 assignments when K <= 4: at most one token per
// thread).
template <int CHUNK, bool ROUTE, bool REGS = false>
__global__ __launch_bounds__(kDispatchThreads) void dispatch_count_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ ntok, int T, int K, int E,
    int32_t* __restrict__ blk_counts, const float* __restrict__ logits, int G,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
    constexpr int kPer = CHUNK / kDispatchThreads;
    static_assert(kPer * kDispatchThreads == CHUNK, "whole rounds");
    __shared__ int s_hist[kMaxExperts];
    __shared__ int s_ids[ROUTE ? CHUNK : 1];
    const long long ntotal = (long long)T * K;
    const long long b0 = (long long)blockIdx.x * CHUNK;
    const long long a0 = b0 + threadIdx.x;
    if (ROUTE) {
        const long long b1 = b0 + CHUNK < ntotal ? b0 + CHUNK : ntotal;
        route_block<REGS>(logits, G, K, moe_valid_tokens(ntok, T), b0, b1, s_ids, ids_out, w_out);
    }
    int v[kPer];   // requested together with the valid-token count
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const long long a = a0 + (long long)k * kDispatchThreads;
        v[k] = a < ntotal ? (ROUTE ? s_ids[a - b0] : ids[a]) : -1;
    }
    const long long nvalid = (long long)moe_valid_tokens(ntok, T) * K;
    for (int e = threadIdx.x; e < E; e += blockDim.x) s_hist[e] = 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const long long a = a0 + (long long)k * kDispatchThreads;
        if (a < nvalid && v[k] >= 0 && v[k] < E) atomicAdd(&s_hist[v[k]], 1);  // integer: order-independent
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        blk_counts[(long long)blockIdx.x * E + e] = s_hist[e];
}

// Up to this many histogram rows the scatter blocks sum the rows before
// theirs directly (one launch fewer); above it a scan grid does it once.
constexpr int kScanMinRows = 64;

// Column e of the per-block histograms blk_counts [nblk + 1][E] becomes, in
// place, the exclusive prefix over the blocks (row b = the rows of expert e
// that blocks 0..b-1 hold), and row nblk receives the column total.  One
// workgroup per expert, 256 blocks per pass with a carry.
__global__ __launch_bounds__(256) void dispatch_block_scan_kernel(int32_t* __restrict__ blk_counts,
                                                                  int nblk, int E) {
    __shared__ int s_wave[4];
    const int e = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int carry = 0;
    for (int b0 = 0; b0 < nblk; b0 += 256) {
        const int b = b0 + tid;
        const int v = b < nblk ? blk_counts[(long long)b * E + e] : 0;
        int incl = v;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int t = __shfl_up(incl, d, 64);
            if (lane >= d) incl += t;
        }
        if (lane == 63) s_wave[wave] = incl;
        __syncthreads();
        int before = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            before += w < wave ? s_wave[w] : 0;
            tot += s_wave[w];
        }
        if (b < nblk) blk_counts[(long long)b * E + e] = carry + before + incl - v;
        carry += tot;
        __syncthreads();
    }
    if (tid == 0) blk_counts[(long long)nblk * E + e] = carry;
}

// SINGLE: one block handles all T*K assignments and builds its own histogram.
// Otherwise block b handles assignments [b*chunk, (b+1)*chunk) and takes its
// start inside each expert and the totals from the nrows histogram rows
// (counted over chunks ratio times smaller): scanned, row b*ratio and row
// nrows of the scanned histograms; else (few rows, no scan grid) the sums of
// the rows before row b*ratio and of all rows.
//
// Wave w of the block owns the contiguous slice of kPer*64 assignments that
// starts at a0 + w*kPer*64 and walks it 64 at a time in increasing order, so
// a wave-local running count per expert gives every assignment its rank among
// the earlier ones of the same expert in that slice.  One pass over the
// per-wave counts (wave order) then turns them into per-wave bases; the rank
// stays in a register until the final write.  The block needs four barriers
// however many rounds it takes.
// ROUTE (single block only): the ids come from the fused router step, which
// writes topk_ids / topk_weights as well.
template <bool SINGLE, bool ROUTE = false, bool REGS = false>
__global__ __launch_bounds__(kDispatchThreads) void dispatch_scatter_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ ntok, int T, int K, int E,
    const int32_t* __restrict__ blk_counts, int nrows, int ratio, bool scanned,
    int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_src, int32_t* __restrict__ token_row,
    const float* __restrict__ logits = nullptr, int G = 0, int32_t* __restrict__ ids_out = nullptr,
    float* __restrict__ w_out = nullptr) {
    static_assert(!ROUTE || SINGLE, "the multi-block form routes in the counting kernel");
    constexpr int kWaves = kDispatchThreads / 64;
    constexpr int kPer = (SINGLE ? kDispatchSingleMax : kDispatchChunk) / kDispatchThreads;
    static_assert(kPer * kDispatchThreads == (SINGLE ? kDispatchSingleMax : kDispatchChunk),
                  "whole rounds");
    __shared__ int s_base[kMaxExperts];            // this block's start inside each expert
    __shared__ int s_scan[kMaxExperts + 1];        // totals -> exclusive offsets
    __shared__ int s_wcnt[kWaves * kMaxExperts];   // per-wave counts -> per-wave bases
    __shared__ int s_wave[kWaves];
    __shared__ int s_ids[ROUTE ? kDispatchSingleMax : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const long long ntotal = (long long)T * K;
    const long long a0 = SINGLE ? 0 : (long long)blockIdx.x * kDispatchChunk;
    const long long a1 = SINGLE ? ntotal : ((a0 + kDispatchChunk < ntotal) ? a0 + kDispatchChunk : ntotal);
    const long long aw = a0 + (long long)wave * kPer * 64 + lane;   // round k adds 64*k
    if (ROUTE) route_block<REGS>(logits, G, K, moe_valid_tokens(ntok, T), 0, ntotal, s_ids, ids_out, w_out);

    // expert of each owned assignment, -1 when dropped or past the end; the
    // ids are requested together with the valid-token count, not after it
    int my_e[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const long long a = aw + 64 * k;
        my_e[k] = a < a1 ? (ROUTE ? s_ids[a] : ids[a]) : -1;
    }
    const long long nvalid = (long long)moe_valid_tokens(ntok, T) * K;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const long long a = aw + 64 * k;
        if (!(a < nvalid && my_e[k] >= 0 && my_e[k] < E)) my_e[k] = -1;
    }
    for (int i = tid; i < kWaves * E; i += blockDim.x) s_wcnt[i] = 0;
    __syncthreads();

    // 1. wave-local ranks and per-wave counts; each wave touches only its own
    //    row of s_wcnt, and a wave's LDS accesses take effect in program order
    int my_rank[kPer];
    int* wc = s_wcnt + wave * E;
    const int nbits = moe_expert_bits(E);
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int e = my_e[k];
        const unsigned long long m = moe_match_mask(e, nbits);
        const int before = __popcll(m & below);
        const int run = e >= 0 ? wc[e] : 0;
        my_rank[k] = run + before;
        if (e >= 0 && before == 0) wc[e] = run + __popcll(m);   // lowest lane of its expert
    }
    __syncthreads();

    // 2. per-expert totals and this block's start inside each expert
    for (int e = tid; e < E; e += blockDim.x) {
        if (SINGLE) {
            int tot = 0;
            for (int w = 0; w < kWaves; ++w) tot += s_wcnt[w * E + e];
            s_base[e] = 0;
            s_scan[e] = tot;
        } else {
            if (scanned) {
                s_base[e] = blk_counts[(long long)blockIdx.x * ratio * E + e];
                s_scan[e] = blk_counts[(long long)nrows * E + e];
            } else {   // few rows: sum the rows before this block's first one
                int pre = 0, tot = 0;
                for (int r = 0; r < nrows; ++r) {
                    const int c = blk_counts[(long long)r * E + e];
                    tot += c;
                    pre += r < (int)blockIdx.x * ratio ? c : 0;
                }
                s_base[e] = pre;
                s_scan[e] = tot;
            }
        }
    }
    __syncthreads();

    // 3. exclusive scan of the totals -> expert_offsets; per-wave counts ->
    //    per-wave first rows, in wave order
    moe_block_exclusive_scan(s_scan, E, s_wave);
    if (blockIdx.x == 0)
        for (int e = tid; e <= E; e += blockDim.x) offsets[e] = s_scan[e];
    for (int e = tid; e < E; e += blockDim.x) {
        int run = s_scan[e] + s_base[e];
        for (int w = 0; w < kWaves; ++w) {
            const int c = s_wcnt[w * E + e];
            s_wcnt[w * E + e] = run;
            run += c;
        }
    }
    __syncthreads();

    // 4. scatter
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const long long a = aw + 64 * k;
        if (a < a1) {
            const int e = my_e[k];
            if (e >= 0) {
                const int r = wc[e] + my_rank[k];
                row_src[r] = (int)a;
                token_row[a] = r;
            } else {
                token_row[a] = -1;
            }
        }
    }
}

// x_disp[r, :] = x[row_src[r] / K, :] for r < R = offsets[E]; 16-byte copies.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4* __restrict__ x,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ row_src,
                                                          int K, int E, int vec_per_row,
                                                          uint4* __restrict__ x_disp) {
    const long long R = offsets[E];
    const long long n = R * vec_per_row;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (long long)gridDim.x * blockDim.x) {
        const long long r = i / vec_per_row;
        const int c = (int)(i - r * vec_per_row);
        const long long t = row_src[r] / K;
        x_disp[r * vec_per_row + c] = x[t * vec_per_row + c];
    }
}

}  // namespace

hipError_t launch_dispatch(const Shape& s, const int32_t* ids, const int32_t* ntok,
                           int32_t* offsets, int32_t* row_src, int32_t* token_row,
                           int32_t* blk_counts, hipStream_t st) {
    const int nblk = dispatch_blocks(s);
    if (nblk == 1) {
        hipLaunchKernelGGL(dispatch_scatter_kernel<true>, dim3(1), dim3(kDispatchThreads), 0, st,
                           ids, ntok, s.T, s.K, s.E, nullptr, 1, 1, false, offsets, row_src,
                           token_row, nullptr, 0, nullptr, nullptr);
    } else {
        const bool scanned = nblk > kScanMinRows;
        hipLaunchKernelGGL((dispatch_count_kernel<kDispatchChunk, false>), dim3(nblk),
                           dim3(kDispatchThreads), 0, st, ids, ntok, s.T, s.K, s.E, blk_counts,
                           nullptr, 0, nullptr, nullptr);
        if (scanned)
            hipLaunchKernelGGL(dispatch_block_scan_kernel, dim3(s.E), dim3(256), 0, st, blk_counts,
                               nblk, s.E);
        hipLaunchKernelGGL(dispatch_scatter_kernel<false>, dim3(nblk), dim3(kDispatchThreads), 0,
                           st, ids, ntok, s.T, s.K, s.E, blk_counts, nblk, 1, scanned, offsets,
                           row_src, token_row, nullptr, 0, nullptr, nullptr);
    }
    return hipGetLastError();
}

template <bool REGS>
static void launch_router_dispatch_impl(const Shape& s, const float* logits, int G,
                                        const int32_t* ntok, int32_t* ids, float* wts,
                                        int32_t* offsets, int32_t* row_src, int32_t* token_row,
                                        int32_t* blk_counts, hipStream_t st) {
    const long long n = (long long)s.T * s.K;
    if (n <= kRouteSingleMax) {   // one block routes and dispatches
        hipLaunchKernelGGL((dispatch_scatter_kernel<true, true, REGS>), dim3(1),
                           dim3(kDispatchThreads), 0, st, nullptr, ntok, s.T, s.K, s.E, nullptr, 1,
                           1, false, offsets, row_src, token_row, logits, G, ids, wts);
        return;
    }
    // routed counting over chunks of 4096 / ratio assignments, the scan over
    // those rows, the scatter over 4096-assignment blocks
    const int ratio = route_count_ratio(s.K);
    const int nrows = route_count_rows(s);
    const int nblk = (int)((n + kDispatchChunk - 1) / kDispatchChunk);
    if (ratio == 4)
        hipLaunchKernelGGL((dispatch_count_kernel<kDispatchChunk / 4, true, REGS>), dim3(nrows),
                           dim3(kDispatchThreads), 0, st, nullptr, ntok, s.T, s.K, s.E, blk_counts,
                           logits, G, ids, wts);
    else
        hipLaunchKernelGGL((dispatch_count_kernel<kDispatchChunk, true, REGS>), dim3(nrows),
                           dim3(kDispatchThreads), 0, st, nullptr, ntok, s.T, s.K, s.E, blk_counts,
                           logits, G, ids, wts);
    const bool scanned = nrows > kScanMinRows;
    if (scanned)
        hipLaunchKernelGGL(dispatch_block_scan_kernel, dim3(s.E), dim3(256), 0, st, blk_counts,
                           nrows, s.E);
    hipLaunchKernelGGL(dispatch_scatter_kernel<false>, dim3(nblk), dim3(kDispatchThreads), 0, st,
                       ids, ntok, s.T, s.K, s.E, blk_counts, nrows, ratio, scanned, offsets,
                       row_src, token_row, nullptr, 0, nullptr, nullptr);
}

hipError_t launch_router_dispatch(const Shape& s, const float* logits, int G, const int32_t* ntok,
                                  int32_t* ids, float* wts, int32_t* offsets, int32_t* row_src,
                                  int32_t* token_row, int32_t* blk_counts, hipStream_t st) {
    if (G <= kRouteRegs)
        launch_router_dispatch_impl<true>(s, logits, G, ntok, ids, wts, offsets, row_src,
                                          token_row, blk_counts, st);
    else
        launch_router_dispatch_impl<false>(s, logits, G, ntok, ids, wts, offsets, row_src,
                                           token_row, blk_counts, st);
    return hipGetLastError();
}

hipError_t launch_gather(const Shape& s, const uint16_t* x, const int32_t* offsets,
                         const int32_t* row_src, uint16_t* x_disp, hipStream_t st) {
    const int vec = s.H / 8;
    long long work = (long long)s.cap * vec;
    long long blocks = (work + 255) / 256;
    if (blocks > 4 * kNumCUs * 4) blocks = 4 * kNumCUs * 4;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                       reinterpret_cast<const uint4*>(x), offsets, row_src, s.K, s.E, vec,
                       reinterpret_cast<uint4*>(x_disp));
    return hipGetLastError();
}

}  // namespace moe
