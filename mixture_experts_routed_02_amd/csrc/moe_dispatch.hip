// Local dispatch of top-k routed assignments into a tight, unpadded,
// expert-major batch (TileOps PR #1738 "[Refactor][MoE] Separate dispatched
// expert compute", Summary and Scope): per-expert histogram, exclusive scan
// into expert_offsets (last entry = valid-row count, left on the GPU), and a
// stable scatter that keeps the rows of one expert in increasing assignment
// order a = t*K + j.
//
// Small problems (T*K <= kDispatchSingleMax) run as one 1024-thread block.
// Larger ones run three fixed grids: a per-block histogram into the
// workspace, an exclusive scan of each expert's column of those histograms
// over the blocks (one block per expert; the column total goes to an extra
// row), then the scatter, in which every block reads its own start inside
// each expert and the totals (no atomics across blocks, nothing to reset
// between calls; the work grows linearly with the number of blocks).
// Within a block, ranks among equal experts come from wave64 ballots: one
// ballot per bit of the expert id gives each lane the mask of lanes holding
// its expert, and the lane's rank is the popcount of that mask below it plus
// the count of that expert earlier in the wave's slice; per-wave counts are
// then scanned across waves in LDS.
#include "moe_internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(kDispatchThreads) void dispatch_count_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ ntok, int T, int K, int E,
    int32_t* __restrict__ blk_counts) {
    constexpr int kPer = kDispatchChunk / kDispatchThreads;
    __shared__ int s_hist[kMaxExperts];
    const long long ntotal = (long long)T * K;
    const long long a0 = (long long)blockIdx.x * kDispatchChunk + threadIdx.x;
    int v[kPer];   // requested together with the valid-token count
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const long long a = a0 + (long long)k * kDispatchThreads;
        v[k] = a < ntotal ? ids[a] : -1;
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
// Otherwise block b handles assignments [b*chunk, (b+1)*chunk) and reads its
// start inside each expert (row b of the scanned histograms) and the totals
// (row nblk).
//
// Wave w of the block owns the contiguous slice of kPer*64 assignments that
// starts at a0 + w*kPer*64 and walks it 64 at a time in increasing order, so
// a wave-local running count per expert gives every assignment its rank among
// the earlier ones of the same expert in that slice.  One pass over the
// per-wave counts (wave order) then turns them into per-wave bases; the rank
// stays in a register until the final write.  The block needs four barriers
// however many rounds it takes.
template <bool SINGLE>
__global__ __launch_bounds__(kDispatchThreads) void dispatch_scatter_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ ntok, int T, int K, int E,
    const int32_t* __restrict__ blk_counts, int nblk, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_src, int32_t* __restrict__ token_row) {
    constexpr int kWaves = kDispatchThreads / 64;
    constexpr int kPer = (SINGLE ? kDispatchSingleMax : kDispatchChunk) / kDispatchThreads;
    static_assert(kPer * kDispatchThreads == (SINGLE ? kDispatchSingleMax : kDispatchChunk),
                  "whole rounds");
    __shared__ int s_base[kMaxExperts];            // this block's start inside each expert
    __shared__ int s_scan[kMaxExperts + 1];        // totals -> exclusive offsets
    __shared__ int s_wcnt[kWaves * kMaxExperts];   // per-wave counts -> per-wave bases
    __shared__ int s_wave[kWaves];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const long long ntotal = (long long)T * K;
    const long long a0 = SINGLE ? 0 : (long long)blockIdx.x * kDispatchChunk;
    const long long a1 = SINGLE ? ntotal : ((a0 + kDispatchChunk < ntotal) ? a0 + kDispatchChunk : ntotal);
    const long long aw = a0 + (long long)wave * kPer * 64 + lane;   // round k adds 64*k

    // expert of each owned assignment, -1 when dropped or past the end; the
    // ids are requested together with the valid-token count, not after it
    int my_e[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const long long a = aw + 64 * k;
        my_e[k] = a < a1 ? ids[a] : -1;
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
            s_base[e] = blk_counts[(long long)blockIdx.x * E + e];
            s_scan[e] = blk_counts[(long long)nblk * E + e];
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
                           ids, ntok, s.T, s.K, s.E, nullptr, 1, offsets, row_src, token_row);
    } else {
        hipLaunchKernelGGL(dispatch_count_kernel, dim3(nblk), dim3(kDispatchThreads), 0, st, ids,
                           ntok, s.T, s.K, s.E, blk_counts);
        hipLaunchKernelGGL(dispatch_block_scan_kernel, dim3(s.E), dim3(256), 0, st, blk_counts,
                           nblk, s.E);
        hipLaunchKernelGGL(dispatch_scatter_kernel<false>, dim3(nblk), dim3(kDispatchThreads), 0,
                           st, ids, ntok, s.T, s.K, s.E, blk_counts, nblk, offsets, row_src,
                           token_row);
    }
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
