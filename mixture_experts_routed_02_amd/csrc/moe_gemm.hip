// Grouped BF16 GEMMs of the dispatched-expert MLP on gfx950 MFMA (TileOps PR
// #1738 "[Refactor][MoE] Separate dispatched expert compute", Review
// follow-up: a gate-up grouped GEMM whose epilogue applies the gated
// pointwise op, then a down grouped GEMM; one column mapping and one
// epilogue serve every row policy).
//
// Every kernel here is persistent and fixed-grid.  The tile schedule comes
// from the GPU-resident expert_offsets (tiles = ceil(M_e / BM) * n_tiles per
// expert; an LDS table in the skinny kernels, a per-wave scan in the tiled
// one), so the valid-row count bounds all the work on the device and the same
// launch serves every T_v (graph replay).  Tiles of one expert are numbered
// m-fastest, so the m-tiles that reuse one weight tile run at the same time
// and share it through L2 / MALL.
//
// MFMA operands are "swapped": the weight rows are the A operand (MFMA rows)
// and the dispatched token rows the B operand (MFMA columns), so an
// accumulator lane holds consecutive output columns of one token row.
// v_mfma_f32_16x16x32_bf16 lane layout (gfx950, checked on the device): lane
// l supplies A row l%16 and B column l%16 with 8 k-values each; lane groups
// l/16 = 0..3 cover k blocks of 8; D[4*(l/16)+i][l%16] lands in accumulator
// i.  v_mfma_f32_32x32x16_bf16 (tiled kernel): lane l supplies row l%32 with
// k group l/32; D[(q/4)*8 + (l/32)*4 + q%4][l%32] lands in accumulator q.
//
// gated: W = [E, 2N, Kd] (rows [0,N) gate, [N,2N) up), C = bf16(silu(g)*u) [cap, N]
// plain: W = [E, N, Kd],                                 C = bf16(acc)      [cap, N]
//
// Contents: the skinny kernels (weight-streaming regime, 16-row tiles with
// split-K over the waves; the variants with the dispatch or the combine
// inside), the skinny pack layout and its kernel, the MX skinny kernels
// (MXFP8 / MXFP4 weights dequantized in registers) with the MX quantizer and
// dequantizer, and the tiled kernel (LDS-staged 192x256 / 128 / 64-row tiles
// for the MFMA-bound and prefill regimes), then the host launchers and the
// plan choice.
#include "moe_internal.h"

#include <cmath>
#include <mutex>

namespace moe {
namespace {

// silu(z) = z / (1 + exp(-z)), with the hardware reciprocal (about 1 ulp of
// fp32, far below the bf16 rounding that follows) in place of an IEEE divide
__device__ __forceinline__ float silu_f32(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Tile table: s_start[e] = sum_{e' < e} ceil(M_e'/BM) * n_tiles, s_start[E] = total.
template <int BM>
__device__ __forceinline__ int build_tile_table(const int32_t* offsets, int E,
                                                int n_tiles, int* s_start, int* s_wave) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int m = offsets[e + 1] - offsets[e];
        s_start[e] = ((m + BM - 1) / BM) * n_tiles;
    }
    __syncthreads();
    moe_block_exclusive_scan(s_start, E, s_wave);
    return s_start[E];
}

// Largest e with s_start[e] <= tile (s_start[0] = 0 <= tile < s_start[E]).
__device__ __forceinline__ int find_expert(const int* s_start, int E, int tile) {
    int lo = 0, hi = E;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_start[mid] <= tile) lo = mid; else hi = mid;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// Skinny kernel: weight-streaming regime (a handful of rows per expert).
// Tile = 16*RB weight rows x 16 token rows x the whole K, split over the 4
// waves of the workgroup (contiguous k ranges), reduced through LDS in wave
// order.  gated: the 16*RB weight rows are 8*RB gate rows and the 8*RB
// matching up rows, so a tile produces 8*RB output columns (the gate-up GEMM
// uses RB = 1: 32-row gated tiles, which halve the token-row loads per weight
// byte, measured no faster); plain: 16*RB output columns (the down GEMM uses
// RB = 2 so that one token's tiles fill the resident workgroups in one
// round).  Each wave keeps two blocks of weights
// (8 KB) in flight: the next block is loaded while the current one is
// multiplied.  Blocks of 4 k-steps (rather than 8) keep the kernel under 128
// VGPRs, so 4 workgroups fit per CU: measured 2-3% faster on the decode
// workloads than 3 workgroups with twice the bytes in flight each.  Token rows
// past the expert's valid rows load a valid row (no branches) and are left as
// they are: MFMA output column j depends on token row j alone, and the
// epilogues write only the valid rows (zeroing them in registers made the
// loads wait early; 1-2% slower on the MXFP8 decode shapes).
// ---------------------------------------------------------------------------
// One-use weight loads.  NT (the skinny pack layout, where each wave's load
// is one contiguous 1 KB block of whole cache lines): with the non-temporal
// hint, so the streamed weights do not displace the token rows and
// partial sums in L2; measured (cold, 32 routing draws, bit-identical) 10%
// faster at decode T = 8, 32 and 128, 5% at T = 1.  Row-major weights stay
// plain: there one load covers 64 bytes of each of 16 rows, half a line, and
// the hint made the same workloads 12-25% slower (15-28% with it only on the
// load that completes each line).
template <bool NT>
__device__ __forceinline__ moe_bf16x8 stream_load(const moe_bf16x8* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// Tile epilogue of the skinny kernels: the four waves' partial sums of the
// tile (accumulator i of lane l in block rb = tile row 16*rb + 4*(l/16) + i,
// token row l%16) are added in wave order through LDS; gated tiles write
// bf16(silu(g) * u) for their 8*RB columns, plain tiles bf16(y) for their
// 16*RB columns.  PACKED_GROUPS: the tile's 16-row blocks are packed groups
// of 8 gate rows and the matching 8 up rows (else a gated tile holds its
// gate rows first, then the matching up rows).  Gated tiles store column
// pairs as 32-bit words; COHERENT makes those device-scope atomic stores
// (visible to every XCD without an L2 writeback).  Ends with a barrier, so
// s_red is free again.
template <bool GATED, int RB, bool PACKED_GROUPS = false, bool COHERENT = false>
__device__ __forceinline__ void skinny_epilogue(const moe_f32x4 (&acc)[RB], float* s_red,
                                                uint16_t* __restrict__ C, int N, int r0,
                                                int mrows, int n_tile) {
    constexpr int COLS = GATED ? 8 * RB : 16 * RB;
    constexpr int RED_ROWS = 16 * RB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    auto red = [&](int w, int row, int m) -> float& { return s_red[(w * RED_ROWS + row) * 17 + m]; };
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) red(wave, rb * 16 + 4 * lg + i, li) = acc[rb][i];
    __syncthreads();
    if (GATED) {
        constexpr int PAIRS = COLS / 2;
        for (int o = tid; o < 16 * PAIRS; o += 256) {
            const int m = o / PAIRS, c0 = 2 * (o % PAIRS);
            if (m < mrows) {
                uint32_t v = 0;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int c = c0 + j;
                    float g = 0.f, u = 0.f;
                    // packed weights: the tile's 16-row groups each hold 8
                    // gate rows and the matching 8 up rows; row-major: the
                    // tile's gate rows come first, then the matching up rows
                    const int rg = PACKED_GROUPS ? (c >> 3) * 16 + (c & 7) : c;
                    const int ru = PACKED_GROUPS ? rg + 8 : COLS + c;
#pragma unroll
                    for (int w = 0; w < 4; ++w) { g += red(w, rg, m); u += red(w, ru, m); }
                    v |= (uint32_t)moe_f32_to_bf16(silu_f32(g) * u) << (16 * j);
                }
                uint32_t* dst = reinterpret_cast<uint32_t*>(C + (size_t)(r0 + m) * N + n_tile * COLS + c0);
                if (COHERENT)
                    __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                else
                    *dst = v;
            }
        }
    } else {
        const int m = tid >> 4, c = tid & 15;
        if (m < mrows) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                float y = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) y += red(w, rb * 16 + c, m);
                C[(size_t)(r0 + m) * N + n_tile * COLS + rb * 16 + c] = moe_f32_to_bf16(y);
            }
        }
    }
    __syncthreads();
}

// RB = 16-row weight blocks per tile (1 or 2; gated tiles use 1).  Blocks of
// U k-steps keep RB * U KB of weights in flight per wave and per buffer.
// offsets and rows may point to global memory or LDS; s_red is
// [4 waves][16*RB rows][17].  PACKED: W is in the skinny pack layout (see
// skinny_pack_kernel), so a wave's load of one k-step is 1 KB contiguous.
// COHERENT: the epilogue's stores of C are device-scope atomic stores.
template <bool GATED, int RB, bool PACKED = false, bool COHERENT = false>
__device__ __forceinline__ void skinny_tiles(const uint16_t* __restrict__ A, const int32_t* rows,
                                             int topk, const int32_t* offsets,
                                             const uint16_t* __restrict__ W,
                                             uint16_t* __restrict__ C, int E, int Kd, int N,
                                             int* s_start, int* s_wave, float* s_red) {
    static_assert(RB == 1 || RB == 2, "tile rows");
    constexpr int BM = 16;
    constexpr int U = 4 / RB;                      // k-steps (of 32) per block
    constexpr int COLS = GATED ? 8 * RB : 16 * RB;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int n_tiles = N / COLS;
    const int w_rows = GATED ? 2 * N : N;
    const int total = build_tile_table<BM>(offsets, E, n_tiles, s_start, s_wave);

    const int ksteps = Kd / 32;
    const int ks0 = (wave * ksteps) / 4, ks1 = ((wave + 1) * ksteps) / 4;
    const int nblk = (ks1 - ks0) / U;              // full blocks; the rest is a tail
    constexpr int WS = PACKED ? 64 : 4;            // 16-byte pieces between k-steps of a lane

    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const int e = find_expert(s_start, E, tile);
        const int row0 = offsets[e];
        const int me = offsets[e + 1] - row0;
        const int mt = (me + BM - 1) / BM;
        const int local = tile - s_start[e];
        const int m_tile = local % mt, n_tile = local / mt;
        const int r0 = row0 + m_tile * BM;
        const int mrows = (me - m_tile * BM) < BM ? (me - m_tile * BM) : BM;

        const moe_bf16x8* wp[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            if (PACKED) {   // 16-row group n_tile (gated) or n_tile * RB + rb (plain)
                const size_t grp = (size_t)e * (w_rows / 16) + (GATED ? n_tile : n_tile * RB + rb);
                wp[rb] = reinterpret_cast<const moe_bf16x8*>(W) + (grp * ksteps + ks0) * 64 + lane;
            } else {
                const int tr = rb * 16 + li;   // gated: rows [0, COLS) gate, then the matching up rows
                const int wrow = !GATED ? n_tile * COLS + tr
                               : tr < COLS ? n_tile * COLS + tr : N + n_tile * COLS + (tr - COLS);
                wp[rb] = reinterpret_cast<const moe_bf16x8*>(
                    W + ((size_t)e * w_rows + wrow) * (size_t)Kd + (size_t)ks0 * 32 + lg * 8);
            }
        }

        moe_bf16x8 wa[RB][U], wb[RB][U], xa[U], xb[U];
        auto load_w = [&](moe_bf16x8 (*wv)[U], int b) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int u = 0; u < U; ++u) wv[rb][u] = stream_load<PACKED>(wp[rb] + (b * U + u) * WS);
        };
        // first weight block before the (dependent) row lookup
        if (nblk > 0) load_w(wa, 0);
        const bool mvalid = li < mrows;
        const int rr = r0 + (mvalid ? li : 0);
        const long long arow = rows ? (long long)(rows[rr] / topk) : (long long)rr;
        const moe_bf16x8* ap = reinterpret_cast<const moe_bf16x8*>(
            A + (size_t)arow * Kd + (size_t)ks0 * 32 + lg * 8);
        auto load_x = [&](moe_bf16x8* xv, int b) {
#pragma unroll
            for (int u = 0; u < U; ++u) xv[u] = ap[(b * U + u) * 4];
        };
        moe_f32x4 acc[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb] = (moe_f32x4){0.f, 0.f, 0.f, 0.f};
        auto mma = [&](moe_bf16x8 (*wv)[U], const moe_bf16x8* xv) {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[rb][u], xv[u], acc[rb], 0, 0, 0);
        };
        if (nblk > 0) load_x(xa, 0);
        int b = 0;
        for (; b + 2 <= nblk; b += 2) {
            load_w(wb, b + 1);
            load_x(xb, b + 1);
            mma(wa, xa);
            if (b + 2 < nblk) {
                load_w(wa, b + 2);
                load_x(xa, b + 2);
            }
            mma(wb, xb);
        }
        if (b < nblk) mma(wa, xa);
        for (int ks = ks0 + nblk * U; ks < ks1; ++ks) {   // tail k-steps
            const int o = (ks - ks0) * 4;
            const moe_bf16x8 xv = ap[o];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(stream_load<PACKED>(wp[rb] + (ks - ks0) * WS), xv,
                                                                  acc[rb], 0, 0, 0);
        }

        skinny_epilogue<GATED, RB, false, COHERENT>(acc, s_red, C, N, r0, mrows, n_tile);
    }
}

template <bool GATED, int RB, bool PACKED = false>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ row_src, int topk,
    const int32_t* __restrict__ offsets, const uint16_t* __restrict__ W,
    uint16_t* __restrict__ C, int E, int Kd, int N) {
    __shared__ int s_start[kMaxExperts + 1];
    __shared__ int s_wave[4];
    __shared__ float s_red[4 * 16 * RB * 17];
    skinny_tiles<GATED, RB, PACKED>(A, row_src, topk, offsets, W, C, E, Kd, N, s_start, s_wave,
                                    s_red);
}

// Expert slots of the tiny down kernels: the experts that hold rows, in
// expert order (at most kTinyRows of them): s_e = expert, s_r0 = first row,
// s_m = rows; *s_ne = their number.  Ends with a barrier.
__device__ __forceinline__ void tiny_expert_slots(const int32_t* __restrict__ offsets, int E,
                                                  int* s_e, int* s_r0, int* s_m, int* s_ne) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (wave == 0) {
        int base = 0;
        for (int c = 0; c * 64 < E; ++c) {
            const int e = c * 64 + lane;
            const int m = e < E ? offsets[e + 1] - offsets[e] : 0;
            const unsigned long long has = __ballot(m > 0);
            const int slot = base + __popcll(has & ((1ull << lane) - 1ull));
            if (m > 0 && slot < kTinyRows) {
                s_e[slot] = e;
                s_r0[slot] = offsets[e];
                s_m[slot] = m;
            }
            base += __popcll(has);
        }
        if (lane == 0) *s_ne = base < kTinyRows ? base : kTinyRows;
    }
    __syncthreads();
}

// End of the tiny down kernels, after every wave stored its partial sums in
// s_part [slot][wave][weight row][17]: y = the four partials added in wave
// order, rounded to bf16 into s_y [slot][token row][16]; then
// out[t, n0 + c] = bf16( sum_j w[t,j] * y[token_row[t*K+j]][c] ), j increasing
// (the combine kernel's arithmetic).
__device__ __forceinline__ void tiny_combine(int ne, const int* s_r0, const float* s_part,
                                             uint16_t* s_y, const int32_t* __restrict__ token_row,
                                             const float* __restrict__ wts,
                                             const int32_t* __restrict__ ntok, int T, int topk,
                                             int N, int n0, uint16_t* __restrict__ out) {
    const int tid = threadIdx.x;
    for (int idx = tid; idx < ne * 256; idx += 256) {
        const int i = idx >> 8, c = (idx >> 4) & 15, m = idx & 15;
        float y = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) y += s_part[((i * 4 + w) * 16 + c) * 17 + m];
        s_y[(i * 16 + m) * 16 + c] = moe_f32_to_bf16(y);
    }
    __syncthreads();
    const int tv = moe_valid_tokens(ntok, T);
    for (int idx = tid; idx < tv * 16; idx += 256) {
        const int t = idx >> 4, c = idx & 15;
        float acc1 = 0.f;
        for (int j = 0; j < topk; ++j) {
            const int r = token_row[(size_t)t * topk + j];
            if (r < 0) continue;
            int i = 0;
            while (i + 1 < ne && r >= s_r0[i + 1]) ++i;
            const float yv = moe_bf16_to_f32(s_y[(i * 16 + (r - s_r0[i])) * 16 + c]);
            acc1 = fmaf(wts[(size_t)t * topk + j], yv, acc1);
        }
        out[(size_t)t * N + n0 + c] = moe_f32_to_bf16(acc1);
    }
}

// ---------------------------------------------------------------------------
// Down GEMM and weighted combine in one kernel for tiny batches (T*K <=
// kTinyRows, so at most kTinyRows experts hold rows and none holds more than
// 16).  Workgroup b owns output columns [16b, 16b+16): for every expert with
// rows it streams those 16 rows of W_down over the whole K, split over the 4
// waves with the skinny kernel's k ranges, blocks and MFMA order (one expert
// after the other, the next block always in flight), reduces the four
// partial sums in wave order, rounds y to bf16 in LDS, and forms
// out[t, cols] for every valid token with the combine kernel's arithmetic.
// The result is bit-identical to the down GEMM followed by the combine, with
// one launch fewer and no y rows through memory.  Needs the per-wave k range
// to be whole blocks of 8 k-steps (I % 1024 == 0).
// ---------------------------------------------------------------------------
// The body, for output columns [16*cb, 16*cb+16).  mid() runs after the
// first block of weights is requested and before the first token rows are
// (the single-launch forward puts its grid barrier there, so the first
// weights are already in flight when the rows of h become readable).
// COHERENT: the rows of A are read with device-scope atomic loads (64-bit),
// which see stores made by other XCDs without an L2 invalidate.  LDS:
// s_e, s_r0, s_m [kTinyRows], s_ne, s_part [kTinyRows][4][16][17] floats,
// s_y [kTinyRows][16][16].
template <bool PACKED, bool COHERENT, typename MID>
__device__ __forceinline__ void tiny_down_combine(
    const uint16_t* __restrict__ A, const int32_t* offsets, const uint16_t* __restrict__ W, int E,
    int Kd, int N, const int32_t* __restrict__ token_row, const float* __restrict__ wts,
    const int32_t* __restrict__ ntok, int T, int topk, uint16_t* __restrict__ out, int cb,
    int* s_e, int* s_r0, int* s_m, int* s_ne, float* s_part, uint16_t* s_y, MID mid) {
    constexpr int U = 8;   // 16 KB of weights in flight per wave
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int n0 = cb * 16;

    tiny_expert_slots(offsets, E, s_e, s_r0, s_m, s_ne);
    const int ne = *s_ne;

    const int ksteps = Kd / 32;
    const int ks0 = (wave * ksteps) / 4;
    const int nb = ((wave + 1) * ksteps) / 4 - ks0;
    const int nblk = nb / U;                       // whole blocks (checked on the host)
    const int total = ne * nblk;

    constexpr int WS = PACKED ? 64 : 4;   // 16-byte pieces between k-steps of a lane
    auto wptr = [&](int i) {
        if (PACKED)
            return reinterpret_cast<const moe_bf16x8*>(W) +
                   (((size_t)s_e[i] * (N / 16) + cb) * ksteps + ks0) * 64 + lane;
        return reinterpret_cast<const moe_bf16x8*>(
            W + ((size_t)s_e[i] * N + n0 + li) * (size_t)Kd + (size_t)ks0 * 32 + lg * 8);
    };
    auto xptr = [&](int i) {
        const int rr = s_r0[i] + (li < s_m[i] ? li : 0);
        return reinterpret_cast<const moe_bf16x8*>(A + (size_t)rr * Kd + (size_t)ks0 * 32 + lg * 8);
    };
    moe_bf16x8 wa[U], wb[U], xa[U], xb[U];
    auto load_w = [&](moe_bf16x8* wv, int b) {
        const int i = b / nblk, kb = b - i * nblk;
        const moe_bf16x8* wp = wptr(i);
#pragma unroll
        for (int u = 0; u < U; ++u) wv[u] = stream_load<PACKED>(wp + (kb * U + u) * WS);
    };
    auto load_x = [&](moe_bf16x8* xv, int b) {
        const int i = b / nblk, kb = b - i * nblk;
        const moe_bf16x8* ap = xptr(i);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (COHERENT) {
                const uint64_t* q = reinterpret_cast<const uint64_t*>(ap + (kb * U + u) * 4);
                const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const uint64_t both[2] = {lo, hi};
                __builtin_memcpy(&xv[u], both, sizeof(both));
            } else {
                xv[u] = ap[(kb * U + u) * 4];
            }
        }
    };
    auto load = [&](moe_bf16x8* wv, moe_bf16x8* xv, int b) {
        load_w(wv, b);
        load_x(xv, b);
    };
    moe_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto step = [&](const moe_bf16x8* wv, const moe_bf16x8* xv, int b) {
#pragma unroll
        for (int u = 0; u < U; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[u], xv[u], acc, 0, 0, 0);
        if ((b + 1) % nblk == 0) {   // last block of expert slot b / nblk
            const int i = b / nblk;
#pragma unroll
            for (int q = 0; q < 4; ++q) s_part[((i * 4 + wave) * 16 + 4 * lg + q) * 17 + li] = acc[q];
            acc = (moe_f32x4){0.f, 0.f, 0.f, 0.f};
        }
    };
    if (total > 0) load_w(wa, 0);
    mid();
    if (total > 0) load_x(xa, 0);
    int b = 0;
    for (; b + 2 <= total; b += 2) {
        load(wb, xb, b + 1);
        step(wa, xa, b);
        if (b + 2 < total) load(wa, xa, b + 2);
        step(wb, xb, b + 1);
    }
    if (b < total) step(wa, xa, b);
    __syncthreads();
    tiny_combine(ne, s_r0, s_part, s_y, token_row, wts, ntok, T, topk, N, n0, out);
}

template <bool PACKED>
__global__ __launch_bounds__(256) void down_combine_tiny_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ offsets,
    const uint16_t* __restrict__ W, int E, int Kd, int N,
    const int32_t* __restrict__ token_row, const float* __restrict__ wts,
    const int32_t* __restrict__ ntok, int T, int topk, uint16_t* __restrict__ out) {
    __shared__ int s_e[kTinyRows], s_r0[kTinyRows], s_m[kTinyRows];
    __shared__ int s_ne;
    __shared__ float s_part[kTinyRows][4][16][17];   // [expert slot][wave][weight row][token row]
    __shared__ uint16_t s_y[kTinyRows][16][16];      // [expert slot][token row][column]
    tiny_down_combine<PACKED, false>(A, offsets, W, E, Kd, N, token_row, wts, ntok, T, topk, out,
                              (int)blockIdx.x, s_e, s_r0, s_m, &s_ne, &s_part[0][0][0][0],
                              &s_y[0][0][0], [] {});
}

// The dispatch of the fused kernels: counts, scans and ranks the T*K (<=
// kFusedDispatchMax) assignments in LDS (s_off: exclusive expert offsets,
// s_off[E] = valid rows; s_rows: row -> assignment); workgroup 0 also
// publishes expert_offsets, row_src and token_row (and, if s_trow is given,
// every workgroup keeps its own LDS copy of token_row).  The ids are read once,
// into registers, together with the valid-token count; wave w ranks the
// contiguous slice of 256 assignments starting at 256*w with per-bit ballot
// masks and a wave-local running count per expert, and the per-wave counts
// double as the histogram.  Ends with a barrier.
__device__ __forceinline__ void fused_dispatch(const int32_t* __restrict__ ids,
                                               const int32_t* __restrict__ ntok, int T, int topk,
                                               int E, int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ row_src,
                                               int32_t* __restrict__ token_row, int* s_off,
                                               int* s_wc, int* s_rows, int* s_wave,
                                               int* s_trow = nullptr) {
    constexpr int kWaves = 4;
    constexpr int kPer = kFusedDispatchMax / (64 * kWaves);   // assignments per lane
    static_assert(kPer * 64 * kWaves == kFusedDispatchMax, "whole slices");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool publish = blockIdx.x == 0;
    const int ntotal = T * topk;
    const int aw = wave * kPer * 64 + lane;       // round k adds 64*k
    int my_e[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int a = aw + 64 * k;
        my_e[k] = a < ntotal ? ids[a] : -1;
    }
    const int nvalid = moe_valid_tokens(ntok, T) * topk;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int a = aw + 64 * k;
        if (!(a < nvalid && my_e[k] >= 0 && my_e[k] < E)) my_e[k] = -1;
    }
    for (int i = tid; i < kWaves * E; i += blockDim.x) s_wc[i] = 0;
    __syncthreads();

    // wave-local ranks; each wave touches only its own row of s_wc, and a
    // wave's LDS accesses take effect in program order
    int my_rank[kPer];
    int* wc = s_wc + wave * E;
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
    for (int e = tid; e < E; e += blockDim.x) {
        int tot = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) tot += s_wc[w * E + e];
        s_off[e] = tot;
    }
    __syncthreads();
    moe_block_exclusive_scan(s_off, E, s_wave);
    if (publish)
        for (int e = tid; e <= E; e += blockDim.x) offsets[e] = s_off[e];
    for (int e = tid; e < E; e += blockDim.x) {   // per-wave counts -> first rows, wave order
        int run = s_off[e];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int c = s_wc[w * E + e];
            s_wc[w * E + e] = run;
            run += c;
        }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int a = aw + 64 * k;
        if (a < ntotal) {
            const int e = my_e[k];
            const int r = e >= 0 ? wc[e] + my_rank[k] : -1;
            if (r >= 0) s_rows[r] = a;
            if (s_trow) s_trow[a] = r;
            if (publish) {
                token_row[a] = r;
                if (r >= 0) row_src[r] = a;
            }
        }
    }
    __syncthreads();
}

// Gate-up GEMM of the skinny plan with the local dispatch done inside (for
// T*K <= kFusedDispatchMax): every workgroup runs fused_dispatch, then its
// gate-up tiles from that LDS copy.  This saves a launch in the
// latency-bound small-batch regime.
template <bool PACKED>
__global__ __launch_bounds__(256) void gemm_skinny_gateup_dispatch_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ ntok, int T, int topk, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_src, int32_t* __restrict__ token_row,
    const uint16_t* __restrict__ W, uint16_t* __restrict__ C, int Kd, int N) {
    __shared__ int s_off[kMaxExperts + 1];        // totals -> exclusive offsets
    __shared__ int s_wc[4 * kMaxExperts];         // per-wave counts -> per-wave first rows
    __shared__ int s_rows[kFusedDispatchMax];
    __shared__ int s_start[kMaxExperts + 1];
    __shared__ int s_wave[4];
    __shared__ float s_red[4 * 16 * 17];
    fused_dispatch(ids, ntok, T, topk, E, offsets, row_src, token_row, s_off, s_wc, s_rows, s_wave);
    skinny_tiles<true, 1, PACKED>(x, s_rows, topk, s_off, W, C, E, Kd, N, s_start, s_wave, s_red);
}

// ---------------------------------------------------------------------------
// Single-launch forward for tiny batches (TileOps PR #1738, review comments:
// the question of one megakernel for the whole layer; FlashInfer PR #3980,
// kernel API migration notes: the top-k combine reduced inside the kernel).
// One cooperative, persistent launch does what the small-batch path does in
// two: every workgroup runs the dispatch in LDS and its gate-up tiles; a
// grid-wide barrier makes h visible everywhere; then workgroup b does the
// down GEMM and the combine for output columns [16b, 16b+16) (the tiny
// path's arithmetic, so the result is bit-identical to it, with the token ->
// row map taken from the workgroup's own dispatch in LDS, so h is the only
// data that crosses workgroups).  Between arriving at the barrier and waiting
// on it, a workgroup requests its first block of down weights, which do not
// depend on h, so that stream overlaps the end of the gate-up phase.
//
// The barrier: h is the only data that crosses workgroups, and it is
// written with device-scope atomic stores and read with device-scope atomic
// loads, which are coherent across the XCDs' L2 caches by themselves.  So
// the barrier needs no L2 writeback or invalidate (a per-workgroup one
// serializes in each XCD's L2 and costs several microseconds at this grid);
// it only has to order completed stores before later loads.  Arrive: every
// thread waits for its own memory operations to complete, then thread 0
// raises the workgroup's flag to the next generation.  Wait: workgroup 0
// polls every flag, then publishes the generation; the others poll the
// generation.  Flags and generation live in a file-scope device variable
// (zero when the code object loads); the generation only grows, so no reset
// is needed between launches.  Every poll is bounded: past the bound a
// workgroup records a timeout and goes on (the launch then computes garbage,
// and moe_single_launch_status reports it and clears the state) instead of
// hanging.  The host launches the kernel cooperatively, with a grid it has
// checked fits on the device at once.
// ---------------------------------------------------------------------------
constexpr int kMaxSingleGrid = 2048;
struct __attribute__((aligned(256))) BarrierLine {
    unsigned int v;
    unsigned int pad[63];
};
struct GridSync {
    BarrierLine gen, timeouts;
    unsigned int flag[kMaxSingleGrid];
};
__device__ GridSync g_grid_sync;
constexpr unsigned int kBarrierSpins = 1u << 22;   // ~0.3 s of polling

__device__ __forceinline__ unsigned int sync_load(const unsigned int* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Polls *p until it differs from (NE) or equals (!NE) v, within the bound.
template <bool NE>
__device__ __forceinline__ void sync_poll(const unsigned int* p, unsigned int v) {
    unsigned int spins = 0;
    while ((sync_load(p) == v) == NE) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins == kBarrierSpins) {
            __hip_atomic_fetch_add(&g_grid_sync.timeouts.v, 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
    }
}

// Arrive: returns (in *s_gen, LDS) the generation this barrier ends.
__device__ __forceinline__ void grid_arrive(unsigned int* s_gen) {
    __builtin_amdgcn_s_waitcnt(0);   // this thread's stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned int g = sync_load(&g_grid_sync.gen.v);
        *s_gen = g;
        __hip_atomic_store(&g_grid_sync.flag[blockIdx.x], g + 1, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
}

__device__ __forceinline__ void grid_wait(const unsigned int* s_gen, unsigned int nblocks) {
    const unsigned int g = *s_gen;
    if (blockIdx.x == 0) {
        for (unsigned int b = threadIdx.x; b < nblocks; b += blockDim.x)
            sync_poll<false>(&g_grid_sync.flag[b], g + 1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_store(&g_grid_sync.gen.v, g + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (threadIdx.x == 0) {
        sync_poll<true>(&g_grid_sync.gen.v, g);
    }
    __syncthreads();
}

// LDS of the single-launch kernel: the dispatch offsets stay for both phases;
// the rest is the gate-up phase's arrays, then reused by the down phase.
constexpr int kSingleP1Bytes = (4 * kMaxExperts + kFusedDispatchMax + kMaxExperts + 1) * 4 + 4 * 16 * 17 * 4;
constexpr int kSingleP2Bytes = (3 * kTinyRows + 1) * 4 + kTinyRows * 4 * 16 * 17 * 4 + kTinyRows * 16 * 16 * 2;
constexpr int kSingleLds = kSingleP1Bytes > kSingleP2Bytes ? kSingleP1Bytes : kSingleP2Bytes;

template <bool PACKED>
__global__ __launch_bounds__(256, 3) void forward_tiny_single_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ ntok, int T, int topk, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_src, int32_t* __restrict__ token_row,
    const uint16_t* __restrict__ Wgu, uint16_t* __restrict__ h, const uint16_t* __restrict__ Wd,
    const float* __restrict__ wts, uint16_t* __restrict__ out, int H, int I) {
    __shared__ int s_off[kMaxExperts + 1];
    __shared__ int s_wave[4];
    __shared__ int s_trow[kTinyRows];
    __shared__ unsigned int s_gen;
    __shared__ __attribute__((aligned(16))) unsigned char s_mem[kSingleLds];
    // gate-up phase
    int* s_wc = reinterpret_cast<int*>(s_mem);
    int* s_rows = s_wc + 4 * kMaxExperts;
    int* s_start = s_rows + kFusedDispatchMax;
    float* s_red = reinterpret_cast<float*>(s_start + kMaxExperts + 1);
    fused_dispatch(ids, ntok, T, topk, E, offsets, row_src, token_row, s_off, s_wc, s_rows, s_wave,
                   s_trow);
    skinny_tiles<true, 1, PACKED, true>(x, s_rows, topk, s_off, Wgu, h, E, H, I, s_start, s_wave,
                                        s_red);
    grid_arrive(&s_gen);
    // down phase (every LDS read of the gate-up phase is behind its last barrier)
    int* s_e = reinterpret_cast<int*>(s_mem);
    int* s_r0 = s_e + kTinyRows;
    int* s_m = s_r0 + kTinyRows;
    int* s_ne = s_m + kTinyRows;
    float* s_part = reinterpret_cast<float*>(s_ne + 1);
    uint16_t* s_y = reinterpret_cast<uint16_t*>(s_part + kTinyRows * 4 * 16 * 17);
    const int ncb = H / 16;
    if ((int)blockIdx.x < ncb) {
        for (int cb = blockIdx.x; cb < ncb; cb += gridDim.x)
            tiny_down_combine<PACKED, true>(h, s_off, Wd, E, I, H, s_trow, wts, ntok, T, topk, out,
                                            cb, s_e, s_r0, s_m, s_ne, s_part, s_y, [&] {
                                                if (cb == (int)blockIdx.x) grid_wait(&s_gen, gridDim.x);
                                            });
    } else {
        grid_wait(&s_gen, gridDim.x);
    }
}

template <bool PACKED>
static hipError_t launch_tiny_single(const Shape& s, const uint16_t* x, const int32_t* ids,
                                     const int32_t* ntok, int32_t* offsets, int32_t* row_src,
                                     int32_t* token_row, const uint16_t* Wgu, uint16_t* h,
                                     const uint16_t* Wd, const float* w, uint16_t* out,
                                     int grid, hipStream_t st) {
    int T = s.T, K = s.K, E = s.E, H = s.H, I = s.I;
    void* args[] = {(void*)&x, (void*)&ids, (void*)&ntok, (void*)&T, (void*)&K, (void*)&E,
                    (void*)&offsets, (void*)&row_src, (void*)&token_row, (void*)&Wgu, (void*)&h,
                    (void*)&Wd, (void*)&w, (void*)&out, (void*)&H, (void*)&I};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&forward_tiny_single_kernel<PACKED>),
                                      dim3(grid), dim3(256), args, 0, st);
}

// ---------------------------------------------------------------------------
// MXFP8 weights (FlashInfer PR #3980: the MXFP8 MegaMoE backend; its combine
// wire names the format, 32 e4m3 values sharing one e8m0 scale).  The skinny
// kernels again, streaming 1-byte OCP e4m3 codes plus one scale byte per 32
// k-values of a weight row, i.e. about half the bytes of bf16 weights, and
// dequantizing in registers: v_cvt_scalef32_pk_bf16_fp8 turns two codes into
// two bf16 values times 2^(s - 127), which is exact for the scales the
// quantizer produces (the product of a 4-bit-significand value and a power
// of two inside bf16's range), so the MFMA sees the dequantized weights
// exactly and accumulates in fp32 as the bf16 path does.
//
// k order.  A lane loads 16 consecutive codes of its weight row, k = 64*seg +
// 16*lg + (0..15), and the matching 16 token values as two 16-byte pieces.
// MFMA step s of the segment takes codes 8s..8s+7 of every lane group, so an
// instruction sums over k = 64*seg + 16*g + 8*s + (0..7), g = 0..3: both
// operands use the same map, and every k of the segment is summed once.  The
// scale of lane group lg is the one of 32-block 2*seg + lg/2; one 16-bit load
// per segment brings both of the segment's scales.
// ---------------------------------------------------------------------------
typedef __bf16 moe_bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));

// MX code loads of the skinny kernels.  NT (the skinny pack layout: each
// wave's load is one contiguous 1 KB block of whole lines): with the
// non-temporal hint, as for bf16 weights (stream_load).  Measured (cold, 32
// routing draws, bit-identical) at decode T = 8 / 32 / 128: MXFP8 6-8%,
// MXFP4 3-5% faster.  Row-major codes stay plain (partial lines per load).
template <bool NT>
__device__ __forceinline__ moe_u32x4 code_load(const moe_u32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// Scale operand of v_cvt_scalef32_*: an fp32 whose exponent field holds the
// e8m0 code (gfx950 reads the scale from those bits).
__device__ __forceinline__ float mx_scale_operand(uint32_t code) { return __uint_as_float(code << 23); }

// 8 e4m3 codes (w0: codes 0-3, w1: codes 4-7, lowest byte first) -> 8 bf16
__device__ __forceinline__ moe_bf16x8 mx_dequant8(uint32_t w0, uint32_t w1, float scale) {
    union {
        moe_bf16x2 p[4];
        moe_bf16x8 v;
    } r;
    r.p[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, false);
    r.p[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, true);
    r.p[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, false);
    r.p[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, true);
    return r.v;
}

// 8 e2m1 codes (4 bytes, the lower nibble of a byte first) -> 8 bf16
__device__ __forceinline__ moe_bf16x8 mx_dequant8_fp4(uint32_t w, float scale) {
    union {
        moe_bf16x2 p[4];
        moe_bf16x8 v;
    } r;
    r.p[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
    r.p[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
    r.p[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
    r.p[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
    return r.v;
}

// The two code formats of the MX skinny kernels.  Either way a lane loads 16
// bytes of codes per segment and a wave 64 bytes of every weight row, so the
// code addressing is the same; what differs is how many k-values those bytes
// hold (G per lane, SEG per wave), the MFMA steps they feed, and which of the
// segment's scale bytes belongs to the lane.
//   FMT 8 (e4m3):  G = 16, SEG = 64,  2 steps; scales of a segment: 2 bytes
//                  (one 16-bit load), lane group lg takes byte lg / 2
//   FMT 4 (e2m1):  G = 32, SEG = 128, 4 steps; scales of a segment: 4 bytes
//                  (one 32-bit load), lane group lg takes byte lg
// Step s of a segment takes the lane's codes 8s..8s+7, so an MFMA sums over
// k = SEG*seg + G*g + 8*s + (0..7), g = 0..3, and the token operand is loaded
// in the same k order (G/8 16-byte pieces per lane and segment).
template <int FMT>
struct MxFmt;
template <>
struct MxFmt<8> {
    static constexpr int G = 16, SEG = 64, STEPS = 2, SCALES = 2;
    typedef uint16_t scale_t;
    __device__ static int scale_shift(int lg) { return 8 * (lg >> 1); }
    __device__ static moe_bf16x8 dequant(const moe_u32x4& q, int s, float scale) {
        return s == 0 ? mx_dequant8(q[0], q[1], scale) : mx_dequant8(q[2], q[3], scale);
    }
};
template <>
struct MxFmt<4> {
    static constexpr int G = 32, SEG = 128, STEPS = 4, SCALES = 4;
    typedef uint32_t scale_t;
    __device__ static int scale_shift(int lg) { return 8 * lg; }
    __device__ static moe_bf16x8 dequant(const moe_u32x4& q, int s, float scale) {
        return mx_dequant8_fp4(q[s], scale);
    }
};

// Tile, block size (segments) and grid of the MX skinny kernels.  Gated
// (gate-up) tiles are 32 weight rows (RB = 2: 16 gate + 16 up rows, or two
// packed 16-row groups), so one set of token registers feeds twice the code
// bytes; plain tiles are 32 rows too when N allows.  From T*K = 128 on,
// MXFP4 gated tiles are 64 rows (RB = 4, 2 workgroups per CU): a segment
// of MXFP4 codes needs twice the token bytes of MXFP8, and 64 rows halve
// them per code byte; below that count 64-row tiles leave CUs idle.  A block
// is 4 segments (MXFP8: 8 KB of codes per wave and buffer at RB = 2, 2
// workgroups per CU) or 2 (MXFP4; 3 workgroups per CU at RB = 2).
// Measured, interleaved and bit-identical, on the 96-expert decode shapes at
// T = 8 .. 128: 32-row gated tiles took MXFP4 15-20% and MXFP8 6-12% below
// 16-row gated tiles (MXFP4 2-segment blocks at 4 x CUs, MXFP8 4-segment
// blocks at 3 x CUs); MXFP4 64-row tiles another 4-6% at T = 32 and 128
// (0% at T = 8, 3-5% slower at T = 1, hence the threshold).  Slower or no
// faster: 3-segment blocks (both formats), 4-segment MXFP4 blocks at 2 x
// CUs, MXFP8 at 3 x CUs (spills), 64-row MXFP8 tiles with 2-segment blocks
// (1-17% slower).  Earlier: 6-segment MXFP8 blocks at 2 x CUs no faster
// than 4; loading the token operand only in the lanes that hold valid rows
// (exec-masked) 0-2% slower on all three formats.  The grid factor is also
// the kernels' waves-per-SIMD bound (__launch_bounds__), so the compiler
// keeps the whole persistent grid resident.
template <int FMT>
constexpr int mx_segs() { return FMT == 8 ? 4 : 2; }
template <int FMT, int RB>
constexpr int mx_grid() { return RB == 4 || FMT == 8 ? 2 : 3; }
// MXFP4 gate-up tiles are 64 weight rows (RB = 4) from this many assignments
// (T*K) on, 32 rows below it, where 64-row tiles would leave CUs idle
constexpr int kMxWideMinAssign = 128;
inline bool mx_wide(int fmt, const Shape& s) { return fmt == 4 && s.T * s.K >= kMxWideMinAssign; }

// Skinny tiles on MX weights: codes Wq [E, rows, Kd * FMT / 8 bytes], scales
// Ws [E, rows, Kd / 32].  Same tile order, k split over the waves (in
// segments), double-buffered blocks and epilogue as skinny_tiles, with RB
// 16-row weight blocks per tile (gated: 2 or 4, plain: 1 or 2); a block is
// US segments.  PACKED: block rb of a tile is 16-row pack group
// n_tile * RB + rb, whose scales are read from the row-major scale rows of
// the same weight rows.
template <int FMT, bool GATED, int RB, bool PACKED = false>
__device__ __forceinline__ void skinny_tiles_mx(const uint16_t* __restrict__ A, const int32_t* rows,
                                                int topk, const int32_t* offsets,
                                                const uint8_t* __restrict__ Wq,
                                                const uint8_t* __restrict__ Ws,
                                                uint16_t* __restrict__ C, int E, int Kd, int N,
                                                int* s_start, int* s_wave, float* s_red) {
    static_assert(RB == 1 || RB == 2 || (GATED && RB == 4), "tile rows");
    typedef MxFmt<FMT> F;
    typedef typename F::scale_t scale_t;
    constexpr int BM = 16;
    constexpr int US = mx_segs<FMT>();              // segments per block
    constexpr int XS = F::G / 8;                   // 16-byte token pieces per lane and segment
    constexpr int COLS = GATED ? 8 * RB : 16 * RB;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar loop bounds
    const int li = lane & 15, lg = lane >> 4;
    const int n_tiles = N / COLS;
    const int w_rows = GATED ? 2 * N : N;
    const int total = build_tile_table<BM>(offsets, E, n_tiles, s_start, s_wave);

    const int nseg = Kd / F::SEG;
    const size_t row_bytes = (size_t)Kd * FMT / 8;
    const int sg0 = (wave * nseg) / 4, sg1 = ((wave + 1) * nseg) / 4;
    const int nblk = (sg1 - sg0) / US;             // full blocks; the rest is a tail
    const int sshift = F::scale_shift(lg);         // this lane group's scale byte
    constexpr int QS = PACKED ? 64 : 4;            // 16-byte pieces between segments of a lane

    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const int e = find_expert(s_start, E, tile);
        const int row0 = offsets[e];
        const int me = offsets[e + 1] - row0;
        const int mt = (me + BM - 1) / BM;
        const int local = tile - s_start[e];
        const int m_tile = local % mt, n_tile = local / mt;
        const int r0 = row0 + m_tile * BM;
        const int mrows = (me - m_tile * BM) < BM ? (me - m_tile * BM) : BM;

        const moe_u32x4* wq[RB];
        const scale_t* wsc[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            // packed: block rb is 16-row group n_tile * RB + rb (gated: 8 gate
            // rows, then the matching 8 up rows); row-major gated: rows
            // [0, COLS) of the tile are gate rows, then the matching up rows
            const int tr = rb * 16 + li, grp16 = n_tile * RB + rb;
            const int wrow = !GATED ? n_tile * COLS + tr
                           : PACKED ? (li < 8 ? 8 * grp16 + li : N + 8 * grp16 + (li - 8))
                           : tr < COLS ? n_tile * COLS + tr : N + n_tile * COLS + (tr - COLS);
            const size_t grow = (size_t)e * w_rows + wrow;
            if (PACKED) {
                const size_t grp = (size_t)e * (w_rows / 16) + grp16;
                wq[rb] = reinterpret_cast<const moe_u32x4*>(Wq) + (grp * nseg + sg0) * 64 + lane;
            } else {
                wq[rb] = reinterpret_cast<const moe_u32x4*>(Wq + grow * row_bytes + (size_t)sg0 * 64 + lg * 16);
            }
            wsc[rb] = reinterpret_cast<const scale_t*>(Ws + grow * (size_t)(Kd / 32)) + sg0;
        }

        moe_u32x4 qa[RB][US], qb[RB][US];
        uint32_t sa[RB][US], sb[RB][US];
        moe_bf16x8 xa[US][XS], xb[US][XS];
        auto load_w = [&](moe_u32x4 (*q)[US], uint32_t (*sc)[US], int b) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int u = 0; u < US; ++u) {
                    q[rb][u] = code_load<PACKED>(&wq[rb][(b * US + u) * QS]);
                    sc[rb][u] = wsc[rb][b * US + u];
                }
        };
        if (nblk > 0) load_w(qa, sa, 0);
        const int rr = r0 + (li < mrows ? li : 0);
        const long long arow = rows ? (long long)(rows[rr] / topk) : (long long)rr;
        const moe_bf16x8* ap = reinterpret_cast<const moe_bf16x8*>(
            A + (size_t)arow * Kd + (size_t)sg0 * F::SEG + lg * F::G);
        auto load_x = [&](moe_bf16x8 (*xv)[XS], int b) {
#pragma unroll
            for (int u = 0; u < US; ++u)
#pragma unroll
                for (int h = 0; h < XS; ++h) xv[u][h] = ap[(b * US + u) * (F::SEG / 8) + h];
        };
        moe_f32x4 acc[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb] = (moe_f32x4){0.f, 0.f, 0.f, 0.f};
        auto seg_mma = [&](const moe_u32x4& q, uint32_t sc, const moe_bf16x8 (&xv)[XS], moe_f32x4& a) {
            const float scale = mx_scale_operand((sc >> sshift) & 0xffu);
#pragma unroll
            for (int st = 0; st < F::STEPS; ++st)
                a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(F::dequant(q, st, scale), xv[st], a, 0, 0, 0);
        };
        auto mma = [&](moe_u32x4 (*q)[US], uint32_t (*sc)[US], moe_bf16x8 (*xv)[XS]) {
#pragma unroll
            for (int u = 0; u < US; ++u)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) seg_mma(q[rb][u], sc[rb][u], xv[u], acc[rb]);
        };
        if (nblk > 0) load_x(xa, 0);
        // Refills inside the loop are unconditional and the last one or two
        // blocks are peeled: a refill under a branch leaves the compiler's
        // wait counts at the join as if it had not been issued, so the next
        // block's multiply would wait for every load in flight (vmcnt(0)).
        // Measured 4-7% faster on the MXFP4 decode shapes, 1-3% on MXFP8,
        // bit-identical; the same change in the bf16 kernels was neutral on
        // packed weights and 3-8% slower on row-major ones, so they keep the
        // conditional refill.
        int b = 0;
        for (; b + 2 < nblk; b += 2) {
            load_w(qb, sb, b + 1);
            load_x(xb, b + 1);
            mma(qa, sa, xa);
            load_w(qa, sa, b + 2);
            load_x(xa, b + 2);
            mma(qb, sb, xb);
        }
        if (b + 1 < nblk) {
            load_w(qb, sb, b + 1);
            load_x(xb, b + 1);
            mma(qa, sa, xa);
            mma(qb, sb, xb);
        } else if (b < nblk) {
            mma(qa, sa, xa);
        }
        for (int sg = sg0 + nblk * US; sg < sg1; ++sg) {   // tail segments
            const int o = sg - sg0;
            moe_bf16x8 xv[XS];
#pragma unroll
            for (int h = 0; h < XS; ++h) xv[h] = ap[o * (F::SEG / 8) + h];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) seg_mma(wq[rb][o * QS], wsc[rb][o], xv, acc[rb]);
        }
        skinny_epilogue<GATED, RB, PACKED>(acc, s_red, C, N, r0, mrows, n_tile);
    }
}

template <int FMT, bool GATED, int RB, bool PACKED = false>
__global__ __launch_bounds__(256, (mx_grid<FMT, RB>())) void gemm_skinny_mx_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ row_src, int topk,
    const int32_t* __restrict__ offsets, const uint8_t* __restrict__ Wq,
    const uint8_t* __restrict__ Ws, uint16_t* __restrict__ C, int E, int Kd, int N) {
    __shared__ int s_start[kMaxExperts + 1];
    __shared__ int s_wave[4];
    __shared__ float s_red[4 * 16 * RB * 17];
    skinny_tiles_mx<FMT, GATED, RB, PACKED>(A, row_src, topk, offsets, Wq, Ws, C, E, Kd, N,
                                            s_start, s_wave, s_red);
}

// Gate-up on MX weights with the dispatch inside (T*K <= kFusedDispatchMax).
template <int FMT, bool PACKED, int RB>
__global__ __launch_bounds__(256, (mx_grid<FMT, RB>())) void gemm_skinny_gateup_dispatch_mx_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ ntok, int T, int topk, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_src, int32_t* __restrict__ token_row,
    const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Ws, uint16_t* __restrict__ C,
    int Kd, int N) {
    __shared__ int s_off[kMaxExperts + 1];
    __shared__ int s_wc[4 * kMaxExperts];
    __shared__ int s_rows[kFusedDispatchMax];
    __shared__ int s_start[kMaxExperts + 1];
    __shared__ int s_wave[4];
    __shared__ float s_red[4 * 16 * RB * 17];
    fused_dispatch(ids, ntok, T, topk, E, offsets, row_src, token_row, s_off, s_wc, s_rows, s_wave);
    skinny_tiles_mx<FMT, true, RB, PACKED>(x, s_rows, topk, s_off, Wq, Ws, C, E, Kd, N, s_start,
                                           s_wave, s_red);
}

// Down GEMM + combine for tiny batches on MX weights: down_combine_tiny_kernel
// with blocks of 256 k-values per wave (4 MXFP8 segments, 4 KB of codes, or 2
// MXFP4 segments, 2 KB); needs whole blocks per wave (I % 1024 == 0).
template <int FMT, bool PACKED = false>
__global__ __launch_bounds__(256) void down_combine_tiny_mx_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ offsets,
    const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Ws, int E, int Kd, int N,
    const int32_t* __restrict__ token_row, const float* __restrict__ wts,
    const int32_t* __restrict__ ntok, int T, int topk, uint16_t* __restrict__ out) {
    typedef MxFmt<FMT> F;
    typedef typename F::scale_t scale_t;
    constexpr int US = FMT == 8 ? 4 : 2;
    constexpr int XS = F::G / 8;
    __shared__ int s_e[kTinyRows], s_r0[kTinyRows], s_m[kTinyRows];
    __shared__ int s_ne;
    __shared__ float s_part[kTinyRows][4][16][17];
    __shared__ uint16_t s_y[kTinyRows][16][16];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar loop bounds
    const int li = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * 16;
    tiny_expert_slots(offsets, E, s_e, s_r0, s_m, &s_ne);
    const int ne = s_ne;

    const int nseg = Kd / F::SEG;
    const size_t row_bytes = (size_t)Kd * FMT / 8;
    const int sg0 = (wave * nseg) / 4;
    const int nblk = (((wave + 1) * nseg) / 4 - sg0) / US;   // whole blocks (checked on the host)
    const int total = ne * nblk;
    const int sshift = F::scale_shift(lg);

    moe_u32x4 qa[US], qb[US];
    uint32_t sa[US], sb[US];
    moe_bf16x8 xa[US][XS], xb[US][XS];
    auto load = [&](moe_u32x4* q, uint32_t* sc, moe_bf16x8 (*xv)[XS], int b) {
        const int i = b / nblk, kb = b - i * nblk;
        const size_t grow = (size_t)s_e[i] * N + n0 + li;
        const moe_u32x4* wp =
            PACKED ? reinterpret_cast<const moe_u32x4*>(Wq) +
                         (((size_t)s_e[i] * (N / 16) + blockIdx.x) * nseg + sg0) * 64 + lane
                   : reinterpret_cast<const moe_u32x4*>(Wq + grow * row_bytes + (size_t)sg0 * 64 + lg * 16);
        const scale_t* sp = reinterpret_cast<const scale_t*>(Ws + grow * (size_t)(Kd / 32)) + sg0;
        const int rr = s_r0[i] + (li < s_m[i] ? li : 0);
        const moe_bf16x8* ap = reinterpret_cast<const moe_bf16x8*>(
            A + (size_t)rr * Kd + (size_t)sg0 * F::SEG + lg * F::G);
#pragma unroll
        for (int u = 0; u < US; ++u) {
            q[u] = code_load<PACKED>(&wp[(kb * US + u) * (PACKED ? 64 : 4)]);
            sc[u] = sp[kb * US + u];
        }
#pragma unroll
        for (int u = 0; u < US; ++u)
#pragma unroll
            for (int h = 0; h < XS; ++h) xv[u][h] = ap[(kb * US + u) * (F::SEG / 8) + h];
    };
    moe_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto step = [&](const moe_u32x4* q, const uint32_t* sc, moe_bf16x8 (*xv)[XS], int b) {
#pragma unroll
        for (int u = 0; u < US; ++u) {
            const float scale = mx_scale_operand((sc[u] >> sshift) & 0xffu);
#pragma unroll
            for (int st = 0; st < F::STEPS; ++st)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(F::dequant(q[u], st, scale), xv[u][st], acc, 0, 0, 0);
        }
        if ((b + 1) % nblk == 0) {   // last block of expert slot b / nblk
            const int i = b / nblk;
#pragma unroll
            for (int r = 0; r < 4; ++r) s_part[i][wave][4 * lg + r][li] = acc[r];
            acc = (moe_f32x4){0.f, 0.f, 0.f, 0.f};
        }
    };
    if (total > 0) load(qa, sa, xa, 0);
    int b = 0;
    for (; b + 2 < total; b += 2) {   // refills unconditional, tail peeled (see skinny_tiles_mx)
        load(qb, sb, xb, b + 1);
        step(qa, sa, xa, b);
        load(qa, sa, xa, b + 2);
        step(qb, sb, xb, b + 1);
    }
    if (b + 1 < total) {
        load(qb, sb, xb, b + 1);
        step(qa, sa, xa, b);
        step(qb, sb, xb, b + 1);
    } else if (b < total) {
        step(qa, sa, xa, b);
    }
    __syncthreads();
    tiny_combine(ne, s_r0, &s_part[0][0][0][0], &s_y[0][0][0], token_row, wts, ntok, T, topk, N, n0, out);
}

// ---------------------------------------------------------------------------
// MX quantization and dequantization of weight rows (OCP MX recipe: the block
// scale is 2^(floor(log2(amax)) - emax), emax being the exponent of the code
// format's largest binade, 8 for e4m3 and 2 for e2m1; codes are v / scale
// rounded to the nearest code value, ties to even, saturated at the largest
// value (448, 6); the code's sign bit is the input's).  Exact integer
// arithmetic on the bf16 bit patterns; one thread per 32-value block.
// ---------------------------------------------------------------------------
// Code of sig * 2^t (sig >= 0 an integer below 2^8) in a format with MB
// mantissa bits, exponent bias BIAS (smallest normal binade 1 - BIAS) and
// largest code MAXC; the sign goes to bit SB.
template <int MB, int BIAS, uint32_t MAXC, int SB>
__device__ __forceinline__ uint32_t mx_code(uint32_t sig, int t, uint32_t sign) {
    if (sig == 0) return sign << SB;
    const int msb = 31 - __clz((int)sig);
    const int L = msb + t;                               // floor(log2(value))
    const int Lmin = 1 - BIAS;                           // smallest normal binade
    const int qe = (L > Lmin ? L : Lmin) - MB;           // exponent of the code spacing
    const int sh = qe - t;                               // value / 2^qe = sig * 2^-sh
    uint32_t n;
    if (sh <= 0) {
        n = sig << (-sh);
    } else if (sh >= 31) {
        n = 0;
    } else {
        n = sig >> sh;
        const uint32_t rem = sig & ((1u << sh) - 1u), half = 1u << (sh - 1);
        if (rem > half || (rem == half && (n & 1u))) ++n;   // nearest, ties to even
    }
    // normal: n in [2^MB, 2^(MB+1)] -> exponent field L + BIAS, mantissa n - 2^MB
    // (n = 2^(MB+1) carries into the next binade); subnormal: the code is n
    uint32_t code = L >= Lmin ? (uint32_t)(((L + BIAS) << MB) + (int)n - (1 << MB)) : n;
    if (L >= Lmin && code > MAXC) code = MAXC;           // saturate
    return code | (sign << SB);
}

// bf16 bits -> (significand, exponent) with |v| = sig * 2^(max(eb, 1) - 134)
template <int FMT>
__global__ __launch_bounds__(256) void mx_quantize_kernel(const uint16_t* __restrict__ w,
                                                          long long nblocks,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
    constexpr int EMAX = FMT == 8 ? 8 : 2;
    const long long blk = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (blk >= nblocks) return;
    typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
    const u16x8* src = reinterpret_cast<const u16x8*>(w + blk * 32);
    uint16_t v[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u16x8 p = src[i];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[8 * i + j] = p[j];
    }
    uint32_t amax = 0;   // magnitude bit patterns order like the magnitudes
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = max(amax, (uint32_t)(v[i] & 0x7FFFu));
    int sc = 0;
    if (amax != 0) {
        const int eb = (int)(amax >> 7);
        const int lg2 = eb ? eb - 127 : (31 - __clz((int)amax)) - 133;   // floor(log2(amax))
        sc = lg2 - EMAX + 127;
        sc = sc < 0 ? 0 : (sc > 254 ? 254 : sc);
    }
    uint32_t c[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const uint32_t m = v[i] & 0x7FFFu, eb = m >> 7, mb = m & 0x7Fu;
        const uint32_t sig = eb ? (128u + mb) : mb;
        const int t = (int)(eb ? eb : 1u) - sc - 7;      // |v| / 2^(sc - 127) = sig * 2^t
        c[i] = FMT == 8 ? mx_code<3, 7, 0x7Eu, 7>(sig, t, v[i] >> 15)
                        : mx_code<1, 1, 0x7u, 3>(sig, t, v[i] >> 15);
    }
    if (FMT == 8) {
        uint32_t out[8] = {};
#pragma unroll
        for (int i = 0; i < 32; ++i) out[i >> 2] |= c[i] << (8 * (i & 3));
        moe_u32x4* dst = reinterpret_cast<moe_u32x4*>(codes + blk * 32);
        dst[0] = (moe_u32x4){out[0], out[1], out[2], out[3]};
        dst[1] = (moe_u32x4){out[4], out[5], out[6], out[7]};
    } else {
        uint32_t out[4] = {};   // value 2i in the low nibble of byte i
#pragma unroll
        for (int i = 0; i < 32; ++i) out[i >> 3] |= c[i] << (4 * (i & 7));
        *reinterpret_cast<moe_u32x4*>(codes + blk * 16) = (moe_u32x4){out[0], out[1], out[2], out[3]};
    }
    scales[blk] = (uint8_t)sc;
}

template <int FMT>
__global__ __launch_bounds__(256) void mx_dequantize_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            long long nblocks,
                                                            uint16_t* __restrict__ w) {
    const long long blk = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (blk >= nblocks) return;
    const float scale = mx_scale_operand(scales[blk]);
    moe_bf16x8* dst = reinterpret_cast<moe_bf16x8*>(w + blk * 32);
    if (FMT == 8) {
        const moe_u32x4* src = reinterpret_cast<const moe_u32x4*>(codes + blk * 32);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const moe_u32x4 q = src[i];
            dst[2 * i] = mx_dequant8(q[0], q[1], scale);
            dst[2 * i + 1] = mx_dequant8(q[2], q[3], scale);
        }
    } else {
        const moe_u32x4 q = *reinterpret_cast<const moe_u32x4*>(codes + blk * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = mx_dequant8_fp4(q[i], scale);
    }
}

// ---------------------------------------------------------------------------
// Skinny pack layout of bf16 expert weights (DeepGEMM PR #394, Summary: expert
// weights stored once in the order the kernel reads them; here the order of
// the skinny kernels' MFMA operand loads).  A weight matrix [E, rows, K] is
// cut into 16-row groups: plain matrices (W_down) take rows 16g .. 16g+15;
// the gated W_gateup [E, 2N, K] takes gate rows 8g .. 8g+7 and the matching
// up rows N+8g .. N+8g+7 (the rows of one gated skinny tile).  Group g of
// expert e is stored as [K/32 k-steps][64 lanes][8 values]: lane l holds row
// l%16 of the group and k-values 32s + 8(l/16) .. +7 of step s, exactly the
// 16 bytes the lane loads for that MFMA step.  One wave load is then 1 KB
// contiguous, and a wave's block of k-steps one contiguous run.  The products
// are the same MFMAs on the same operands: the output is bit-identical.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void skinny_pack_kernel(const uint16_t* __restrict__ w,
                                                          long long pieces, int rows, int Kd,
                                                          int gated, uint16_t* __restrict__ out) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;   // output piece
    if (i >= pieces) return;
    const int ksteps = Kd / 32;
    const int l = (int)(i & 63);
    const long long t = i >> 6;
    const int st = (int)(t % ksteps);
    const long long eg = t / ksteps;                 // e * (rows / 16) + g
    const int groups = rows / 16;
    const long long e = eg / groups;
    const int g = (int)(eg % groups);
    const int li = l & 15, lg = l >> 4;
    const int half = rows / 2;
    const int r = !gated ? 16 * g + li : (li < 8 ? 8 * g + li : half + 8 * g + (li - 8));
    const moe_bf16x8* src = reinterpret_cast<const moe_bf16x8*>(
        w + ((size_t)e * rows + r) * (size_t)Kd + (size_t)st * 32 + lg * 8);
    reinterpret_cast<moe_bf16x8*>(out)[i] = *src;
}

// ---------------------------------------------------------------------------
// Tiled kernel: BM token rows x BN weight rows per tile.  Operands stream
// through LDS rings, 64 k-values (128 bytes of every row) per stage, filled
// by direct global->LDS loads (global_load_lds_dwordx4: no staging
// registers).  A 128-byte row segment is one cache line: measured on the
// device, 1 KiB DMA instructions that cover 8 rows x 128 B move ~1.7x more
// data per CU through the address unit than 16 rows x 64 B, and at this
// kernel's ~128 FLOP per staged byte the address unit is what runs out first.
// The product runs on v_mfma_f32_32x32x16_bf16.
//
// Stage layout: 8-row groups of 1 KiB.  Row r holds its 64-element k-slice
// as eight 16-byte chunks, chunk c stored in slot c ^ f(r % 32),
// f(r) = ((r >> 1) & 3) | ((r >> 2) & 4).  A DMA instruction fills one group
// (lane L writes row L/8, slot L%8, so it fetches chunk (L%8) ^ f); a
// 32x32x16 fragment read takes 32 rows x one chunk.  A ds_read_b128 pass on
// gfx950 serves lanes {0-7,16-23}, {8-15,24-31}, ...: rows of one parity
// among r..r+7 differ in bits 0-1 of f, rows r and r+16 in bit 2, so the
// sixteen lanes of a pass hit sixteen distinct 16-byte bank groups and the
// fragment reads are conflict-free.
//
// Two rings: token stages (SA slots) and weight stages (SW >= SA slots), so
// the weights, which miss L2 more often, are requested further ahead.  LDS
// holds nothing else; the tile table lives in registers.
//
// Pipeline.  Stage d is multiplied as two 32-wide halves 2d and 2d+1; the
// fragments of half h+1 are read from LDS while half h runs its MFMAs (each
// fragment into its own registers right after its last MFMA of half h), so
// every read of stage d is done by the start of half 2d+1.  There, each wave waits for its own
// loads of stage d+1, one barrier tells every wave that stage d+1 has landed
// everywhere and that nobody reads stage d's slots any more; the wave refills
// the token slot with stage d+SA during half 2d+1 and the weight slot with
// stage d+SW during half 2d+2, each refill spread between the MFMAs of its
// half, so that the loads of the eight waves do not arrive at the address
// unit in one burst.  Even halves wait for nothing.  The vmcnt of each wait
// counts the loads this wave issued after the ones it needs.  In the PROD
// instances only waves 0-3 issue loads (twice as many each) and waves 4-7
// only read fragments and multiply; a wave that issued nothing passes its
// vmcnt waits at once, and the barrier still orders every read against the
// next refill.
//
// WGM x WGN waves; each wave owns (BM/WGM) token rows x (BN/WGN) weight rows
// of the tile as 32x32 MFMA sub-tiles (weights = MFMA rows, tokens = MFMA
// columns).  gated: tile rows [0, BN/2) are gate columns n0.. and [BN/2, BN)
// the matching up columns; each wave takes the same column range from both
// halves so gate and up of one output meet in one lane.  Waits on the rings
// are explicit (vmcnt + s_barrier): a full __syncthreads() would also drain
// the loads that are meant to stay in flight.
// ---------------------------------------------------------------------------
constexpr int kBK = 64;   // k-values per stage
constexpr int kMGroup = 8;   // m-tiles per group in the tile walk of a large expert

// LDS per workgroup: all of it when one 8-wave workgroup fills a CU, half
// when two 4-wave ones share it
constexpr int ring_budget(int waves) { return (waves == 8 ? 160 : 80) * 1024; }
// token slots: 3 if both rings can have 3, else 2
constexpr int ring_sa(int a_bytes, int w_bytes, int budget) {
    return 3 * (a_bytes + w_bytes) <= budget ? 3 : 2;
}
// weight slots: what is left, at most 5
constexpr int ring_sw(int a_bytes, int w_bytes, int budget) {
    const int s = (budget - ring_sa(a_bytes, w_bytes, budget) * a_bytes) / w_bytes;
    return s > 5 ? 5 : s;
}

typedef __attribute__((address_space(3))) unsigned char lds_u8;

// 16 bytes per lane from g into LDS at lds_base + 16 * lane (lds_base must be
// wave-uniform).  Written as inline asm so that the compiler does not treat
// the pending LDS writes as aliasing every later LDS read (it would then drain
// the whole ring with vmcnt(0) before each read); the ring's own explicit
// vmcnt waits and barriers order these writes against the reads.  m0 is
// written here only; the kernels below use it for nothing else.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds_base)) : "memory", "m0");
}

// The same with the non-temporal hint, for weight rows that no other tile of
// the launch reads (see gemm_tiled_kernel): they then do not displace the
// token blocks that the expert's column tiles read again from L2.
__device__ __forceinline__ void lds_dma16_nt(const void* g, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds_base)) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p) {
    return (uint32_t)(uintptr_t)(const lds_u8*)p;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
    wait_vmcnt<N>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// LDS writes of this wave done, then a workgroup barrier (no vmcnt drain)
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// chunk swizzle of row r (see above)
__device__ __forceinline__ int ring_swz(int r) { return ((r >> 1) & 3) | ((r >> 2) & 4); }

// MX weight stages (see gemm_tiled_kernel, WF != 16): a 64-value stage of a
// weight row is 64 bytes of e4m3 codes (four 16-byte chunks) or 32 bytes of
// e2m1 codes (two), chunk c of row r stored in slot c ^ swz(r % 32).  The 16
// lanes of a ds_read_b128 pass read one chunk of rows {r..r+7, r+16..r+23},
// which these swizzles put on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int mx8_swz(int r) { return ((r >> 2) & 1) | ((r >> 3) & 2); }
__device__ __forceinline__ int mx4_swz(int r) { return (r >> 4) & 1; }

// Scale bytes of one weight row kept in LDS by the MX tiled kernels: up to
// this many 32-value blocks (K <= 7168).
constexpr int kMxMaxKBlocks = 224;

// Tile table of the tiled kernel, recomputed by each wave from expert_offsets
// when it needs it (no LDS): expert e owns ceil(M_e / BM) * n_tiles logical
// tiles, in expert order.  Lane l looks after experts 64*c + l; a wave scan
// gives each expert's first tile.  Returns the total and, for `tile` < total,
// the owning expert (the largest e whose first tile is <= tile: first tiles
// are non-decreasing, so that is the count of such e, minus one) and its
// first tile.
template <int BM>
__device__ __forceinline__ int wave_tile_lookup(const int32_t* offsets, int E, int n_tiles,
                                                int lane, int tile, int& expert, int& first) {
    int carry = 0, cnt_le = 0, first_v = 0;
    for (int c = 0; c * 64 < E; ++c) {
        const int e = c * 64 + lane;
        int cnt = 0;
        if (e < E) {
            const int m = offsets[e + 1] - offsets[e];
            cnt = ((m + BM - 1) / BM) * n_tiles;
        }
        int v = cnt;   // inclusive scan over the wave
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(v, o);
            if (lane >= o) v += t;
        }
        const int start = carry + v - cnt;
        const unsigned long long le = __ballot(e < E && start <= tile);
        cnt_le += __popcll(le);
        if (le) first_v = __shfl(start, 63 - __clzll(le));   // last expert so far with start <= tile
        carry += __shfl(v, 63);
    }
    expert = __builtin_amdgcn_readfirstlane(cnt_le - 1);
    first = __builtin_amdgcn_readfirstlane(first_v);
    return __builtin_amdgcn_readfirstlane(carry);
}

template <int BM, int BN, int WGM, int WGN, bool GATED, bool SUBSKIP = false, bool PACKED = false,
          int WF = 16, bool PROD = false>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_tiled_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ row_src, int topk,
    const int32_t* __restrict__ offsets, const uint16_t* __restrict__ W,
    uint16_t* __restrict__ C, int E, int Kd, int N, int split,
    const uint8_t* __restrict__ Ws = nullptr) {
    // WF: weight format, 16 = bf16, 8 = MXFP8 (e4m3 codes), 4 = MXFP4 (e2m1
    // codes, two per byte); the MX formats take e8m0 scales Ws [E, rows, Kd/32]
    constexpr bool MX = WF != 16;
    constexpr int NT = 64 * WGM * WGN, NW = NT / 64;  // threads, waves
    constexpr int WM = BM / WGM, WN = BN / WGN;       // per-wave extent
    constexpr int MS = WM / 32, NS = WN / 32;         // 32x32 sub-tiles per wave
    constexpr int COLS = GATED ? BN / 2 : BN;         // output columns per tile
    constexpr int RBW = WF == 16 ? 128 : (WF == 8 ? 64 : 32);   // weight-row bytes per stage
    constexpr int WROWS = 1024 / RBW;                 // weight rows per 1 KiB DMA group
    constexpr int AG = BM / 8, WG = BN / WROWS;       // 1 KiB groups per stage
    // PROD: only waves 0..3 (one per SIMD) issue the ring's DMAs, the other
    // waves only read fragments and multiply (see the launch choice below)
    constexpr int NP = PROD ? 4 : NW;                 // waves that issue DMAs
    constexpr int GA = AG / NP, GW = WG / NP;         // DMA instructions per issuing wave per stage
    constexpr int A_STAGE = AG * 1024, W_STAGE = WG * 1024;
    constexpr int SCL = MX ? BN * kMxMaxKBlocks : 0;  // the tile's scales (MX), bytes
    constexpr int BUDGET = ring_budget(NW) - SCL;
    constexpr int SA = ring_sa(A_STAGE, W_STAGE, BUDGET);
    constexpr int SW = ring_sw(A_STAGE, W_STAGE, BUDGET);
    constexpr int OP = 2 * COLS + 8;                  // epilogue staging pitch, bytes
    constexpr int RINGS = SA * A_STAGE + SW * W_STAGE;
    constexpr int SCL_OFF = RINGS > BM * OP ? RINGS : BM * OP;
    constexpr int LDS = SCL_OFF + SCL;
    // loads issued after the ones a wait needs: at an odd half (stage d+1),
    // and in the prologue (stage 0)
    constexpr int N_STEADY = SW > SA ? (SA - 1) * GW + (SA - 2) * GA : (SA - 2) * (GA + GW);
    constexpr int N_FIRST = SW > SA ? (SA - 1) * (GA + GW) : (SA - 1) * GA + (SA - 2) * GW;
    static_assert(WM % 32 == 0 && WN % 32 == 0 && AG % NW == 0 && WG % NW == 0, "tile shape");
    static_assert(NW % 4 == 0, "a wave's DMA groups share one row-swizzle phase");
    static_assert(!GATED || NS % 2 == 0, "gated tiles pair gate and up sub-tiles");
    static_assert(SA >= 2 && SW >= SA && LDS <= ring_budget(NW), "ring sizes");
    static_assert(!MX || WF == 8 || WF == 4, "MX: e4m3 or e2m1 codes");
    static_assert(N_FIRST < 64 && N_STEADY < 64, "vmcnt range");
    static_assert(!PROD || (WF == 16 && NW == 8 && AG % 4 == 0 && WG % 4 == 0), "issuing waves");

    __shared__ __attribute__((aligned(1024))) unsigned char s_lds[LDS];
    unsigned char* const s_ringA = s_lds;
    unsigned char* const s_ringW = s_lds + SA * A_STAGE;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool producer = wave < NP;
    // token sub-tile index varies slowest across waves, so the waves that stay
    // active on a ragged last m-tile sit on different SIMDs
    const int wm = wave / WGN, wn = wave % WGN;
    const int n_tiles = N / COLS;
    const int w_rows = GATED ? 2 * N : N;
    int e_unused, f_unused;
    const int total = wave_tile_lookup<BM>(offsets, E, n_tiles, lane, 0, e_unused, f_unused);
    const int nk = Kd / kBK;
    const uint32_t ringA0 = lds_addr(s_ringA), ringW0 = lds_addr(s_ringW);

    // XCD-aware order: workgroup b runs on XCD b % 8; give each XCD a
    // contiguous run of logical tiles so neighbouring m-tiles share its L2.
    const int G = gridDim.x;
    const int lb = (G % 8 == 0) ? ((int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8))
                                : (int)blockIdx.x;

    // DMA role of this lane: row lane/8 of a group, slot lane%8.  Group g holds
    // rows 8g..8g+7, i.e. rows 8*(g%4).. of its 32-row block, and g % 4 is
    // wave % 4 for every group this wave fills (g = wave + NP*q).
    const int dma_row = lane >> 3;
    const int dma_chunk = (lane & 7) ^ ring_swz((wave & 3) * 8 + dma_row);
    // MX weight groups: 16 rows x 64 bytes (lane: row lane/4, slot lane%4) or
    // 32 rows x 32 bytes (row lane/2, slot lane%2); a 16-row group's rows are
    // rows 16*(g%2).. of its 32-row block, and g % 2 = wave % 2 for every
    // group this wave fills
    const int wdma_row = WF == 16 ? dma_row : (WF == 8 ? lane >> 2 : lane >> 1);
    const int wdma_chunk = WF == 16 ? dma_chunk
                         : WF == 8 ? (lane & 3) ^ mx8_swz((wave & 1) * 16 + wdma_row)
                                   : (lane & 1) ^ mx4_swz(wdma_row);
    // fragment-read offsets of this lane inside a 32-row token block for the
    // four 16-wide k steps m of a stage: row l%32 and the k-chunk (8 values)
    // that lane group l/32 supplies to MFMA m.  bf16 weights: chunk 2m + l/32
    // on both operands.  MX weights set the k order: a lane group reads 16
    // consecutive codes of its row per half-stage (e4m3: k = 32q + 16g + 0..15
    // for MFMAs 2q, 2q+1) or 32 per stage (e2m1: k = 32g + 0..31 for MFMAs
    // 0..3), so the token chunk of MFMA m is 4(m/2) + 2g + m%2, or 4g + m.
    const int fr = lane & 31, fh = lane >> 5;
    int rd_off[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int ch = WF == 16 ? 2 * s + fh : WF == 8 ? 4 * (s >> 1) + 2 * fh + (s & 1) : 4 * fh + s;
        rd_off[s] = fr * 128 + ((ch ^ ring_swz(fr)) << 4);
    }
    // MX weight fragments: byte offset of this lane's 16 code bytes in its
    // 32-row block for half-stage q (e4m3) / the stage (e2m1)
    int wro[2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
        wro[q] = WF == 8 ? fr * 64 + (((2 * q + fh) ^ mx8_swz(fr)) << 4)
                         : fr * 32 + ((fh ^ mx4_swz(fr)) << 4);
    int ga[MS], gw[NS], wtr[NS];   // byte offsets of this wave's 32-row blocks in a stage
#pragma unroll
    for (int j = 0; j < MS; ++j) ga[j] = (wm * WM + j * 32) * 128;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        int trow;
        if (GATED) trow = (i < NS / 2) ? (wn * (WN / 2) + i * 32)
                                       : (BN / 2 + wn * (WN / 2) + (i - NS / 2) * 32);
        else trow = wn * WN + i * 32;
        gw[i] = trow * RBW;
        wtr[i] = trow;
    }
    const int sp = Kd / 32;                           // scale bytes per weight row (MX)
    const size_t wrow_bytes = (size_t)Kd * WF / 8;    // bytes of one weight row

    // split (many experts): XCDs 0-3 walk the first half of the tile list and
    // XCDs 4-7 the second, each XCD still over contiguous runs, so that the
    // workgroups in flight stream the weights of twice as many experts at
    // once.  Measured: static-capacity layer (128 experts) 8% faster, EP
    // prefill (96) 1.5% faster, Mixtral (8 experts) 1.5% slower, so the host
    // sets it from the expert count (GemmPlan::split).
    int tile0 = lb, tstep = G, tend = total;
    if (split && G % 8 == 0 && total >= 2 * G) {
        const int x = (int)(blockIdx.x % 8), i = (int)(blockIdx.x / 8);
        const int half_total = (total + 1) / 2;
        tile0 = (x >= 4 ? half_total : 0) + (x % 4) * (G / 8) + i;
        tstep = G / 2;
        tend = x >= 4 ? total : half_total;
    }
    for (int tile = tile0; tile < tend; tile += tstep) {
        int e, first;
        wave_tile_lookup<BM>(offsets, E, n_tiles, lane, tile, e, first);
        const int row0 = offsets[e];
        const int me = offsets[e + 1] - row0;
        const int mt = (me + BM - 1) / BM;
        // Non-temporal weight DMAs (PROD instances, few rows per expert): a
        // weight tile of an expert with one m-tile is read by this tile
        // alone, so its DMAs carry the hint and its lines do not displace the
        // token blocks that the expert's column tiles read again from L2.  An
        // expert with several m-tiles has its weight tiles read again by the
        // neighbouring m-tiles, and the hint there made Mixtral 13% and 256
        // rows per expert 19% slower.  Measured against plain DMAs,
        // bit-identical, over two boxes: static capacity 6-9% and EP prefill
        // at 2048 tokens 9-13% faster, at 8192 tokens 0-1%, Zipf-routed
        // prefill at 8192 tokens 2% on average over the seeds (from 1% slower
        // to 4% faster).  Taking the hint on every weight DMA of these
        // instances, with no test per tile, is 2.6% faster on uniform routing
        // but 3% slower on Zipf routing; a second copy of the k loop per case
        // spills.
        const bool w_once = PROD && !MX && __builtin_amdgcn_readfirstlane(mt) == 1;
        const int local = tile - first;
        // An expert's tiles run m-tile fastest, so the 32 consecutive tiles an
        // XCD holds share weight tiles and token blocks.  An expert with more
        // than kMGroup m-tiles (a hot expert under skewed routing) is walked
        // in groups of kMGroup m-tiles, each group over all weight columns
        // before the next, so a window spans about 8 m-tiles x 4 columns
        // instead of one column of all its m-tiles, and its token blocks are
        // not fetched again for every column.  A permutation of the tiles:
        // the output is the same bit for bit.  Measured: Zipf-routed prefill
        // at 8192 tokens 1.6-2.4% faster on the seeds with a hot local expert,
        // the other workloads unchanged.
        int m_tile, n_tile;
        if (mt <= kMGroup) {
            m_tile = local % mt;
            n_tile = local / mt;
        } else {
            const int grp = local / (kMGroup * n_tiles);
            const int gm = mt - grp * kMGroup < kMGroup ? mt - grp * kMGroup : kMGroup;
            const int idx = local - grp * kMGroup * n_tiles;
            n_tile = idx / gm;
            m_tile = grp * kMGroup + idx % gm;
        }
        // The expert's rows, in 32-row units, are split over its mt m-tiles as
        // evenly as whole units allow (heights differ by at most 32 rows and
        // never exceed BM), rather than mt - 1 full tiles and a ragged last
        // one: the m-tiles that share a weight tile and a token block then take
        // about the same time and stay in step, so the blocks they share are
        // fetched once.  Each output row's arithmetic does not depend on its
        // tile, so the result is the same bit for bit.
        const int units = (me + 31) / 32;
        const int ub = units / mt, ux = units % mt;
        const int u0 = m_tile * ub + (m_tile < ux ? m_tile : ux);
        const int r0 = row0 + 32 * u0;
        const int mrows = (me - 32 * u0) < 32 * (ub + (m_tile < ux)) ? (me - 32 * u0)
                                                                       : 32 * (ub + (m_tile < ux));
        // a wave whose token rows all lie past the valid rows skips its MFMAs
        const bool active = wm * WM < mrows;
        // SUBSKIP: the 32-row sub-tiles of this wave that hold valid rows
        // (wave-uniform); the others skip their MFMAs too.  The k loop exists
        // twice: without any test for waves whose sub-tiles all hold rows, and
        // with a test per MFMA for the others, so full tiles pay nothing for it.
        // Instances without PROD (many rows per expert) have a third copy for
        // waves whose last sub-tile alone is empty (an expert's m-tiles of
        // 160 rows, the common height at about 1000 rows per expert), which
        // skips that sub-tile's MFMAs and fragment reads with no test:
        // Mixtral 0.4-0.5% faster on three seeds, bit-identical (the PROD
        // instances have no registers left for a third copy).
        const int jlive = __builtin_amdgcn_readfirstlane((mrows - wm * WM + 31) / 32);

        // global source of each group this wave fills (stage 0): token groups
        // gather rows through row_src (rows past the valid ones repeat the
        // last valid row); weight rows are affine in the group.  PROD keeps
        // the (twice as many) token rows as 32-bit row numbers instead of
        // pointers, to stay within the register budget.
        const int pw = producer ? wave : 0;
        const uint16_t* asrc[PROD ? 1 : GA];
        uint32_t arow_q[PROD ? GA : 1];
#pragma unroll
        for (int q = 0; q < GA; ++q) {
            const int tr = (pw + NP * q) * 8 + dma_row;
            const int rr = r0 + (tr < mrows ? tr : mrows - 1);
            const long long arow = row_src ? (long long)(row_src[rr] / topk) : (long long)rr;
            if constexpr (PROD) arow_q[q] = (uint32_t)arow;
            else asrc[q] = A + (size_t)arow * Kd + dma_chunk * 8;
        }
        auto token_src = [&](int q) -> const uint16_t* {
            if constexpr (PROD) return A + (size_t)arow_q[q] * Kd + dma_chunk * 8;
            else return asrc[q];
        };
        // row-major: lane (dma_row, slot) reads chunk dma_chunk of its row;
        // PACKED (tiled pack layout): the 1 KiB of a group and stage is
        // contiguous and already in slot order, so lane L reads piece L
        const uint16_t* wbase = PACKED ? W + (size_t)e * w_rows * Kd + lane * 8
                                       : W + (size_t)e * w_rows * Kd + (size_t)dma_row * Kd + dma_chunk * 8;
        // MX: byte address of this lane's 16 code bytes (row wdma_row of a group,
        // chunk wdma_chunk), stage 0; PACKED (tiled pack layout of the codes):
        // the 1 KiB of a group and stage is contiguous and in slot order, so
        // lane L reads piece L, and group g's stages start g * WROWS rows'
        // worth of bytes into the expert's block, as row-major rows would
        const unsigned char* wbase_mx =
            PACKED ? reinterpret_cast<const unsigned char*>(W) + (size_t)e * w_rows * wrow_bytes + lane * 16
                   : reinterpret_cast<const unsigned char*>(W) +
                         ((size_t)e * w_rows + wdma_row) * wrow_bytes + wdma_chunk * 16;
        auto wrow0 = [&](int q) {   // first weight row of this wave's weight group q
            const int tr = (pw + NP * q) * WROWS;
            if (GATED) return (tr < BN / 2) ? (n_tile * (BN / 2) + tr) : (N + n_tile * (BN / 2) + tr - BN / 2);
            return n_tile * BN + tr;
        };
        // DMA number q of a refill pair: tokens first (q < GA), then weights
        auto issue_one = [&](int sa, int sw, int q) {
            if (PROD && !producer) return;
            if (q < GA) {
                lds_dma16(token_src(q < GA ? q : 0) + (size_t)sa * kBK,
                          ringA0 + (sa % SA) * A_STAGE + (pw + NP * q) * 1024);
            } else {
                const int qw = q - GA;
                const uint32_t dst = ringW0 + (sw % SW) * W_STAGE + (pw + NP * qw) * 1024;
                if constexpr (MX)
                    lds_dma16(wbase_mx + (size_t)wrow0(qw) * wrow_bytes + (size_t)sw * (PACKED ? 1024 : RBW),
                              dst);
                else {  // packed: group wrow0/8 holds Kd/64 stages of 512 values each
                    const uint16_t* src = PACKED ? wbase + (size_t)wrow0(qw) * Kd + (size_t)sw * 512
                                                 : wbase + (size_t)wrow0(qw) * Kd + (size_t)sw * kBK;
                    if constexpr (PROD && !MX) {
                        if (w_once) lds_dma16_nt(src, dst);
                        else lds_dma16(src, dst);
                    } else {
                        lds_dma16(src, dst);
                    }
                }
            }
        };

        moe_f32x16 acc[NS][MS];
#pragma unroll
        for (int i = 0; i < NS; ++i)
#pragma unroll
            for (int j = 0; j < MS; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

        moe_bf16x8 fw[2][NS], fa[2][MS];
        // fragments of half h (stage h/2, k steps 2*(h%2) and 2*(h%2)+1)
        auto read_a = [&](int h, int sk, int j) {
            const unsigned char* st = s_ringA + ((h >> 1) % SA) * A_STAGE;
            fa[sk][j] = *reinterpret_cast<const moe_bf16x8*>(st + ga[j] + rd_off[2 * (h & 1) + sk]);
        };
        auto read_w = [&](int h, int sk, int i) {
            const unsigned char* st = s_ringW + ((h >> 1) % SW) * W_STAGE;
            fw[sk][i] = *reinterpret_cast<const moe_bf16x8*>(st + gw[i] + rd_off[2 * (h & 1) + sk]);
        };
        // MX weights: the lane's 16 code bytes for half h (e4m3) or for stage
        // h/2 (e2m1), and the two scale bytes of its row for stage d (blocks
        // 2d, 2d+1), read a half ahead; dequant_w turns them into the half's
        // two bf16 fragments at its start
        moe_u32x4 wraw[MX ? NS : 1];
        uint32_t wsc[MX ? NS : 1];
        auto read_w_raw = [&](int h, int i) {
            const unsigned char* st = s_ringW + ((h >> 1) % SW) * W_STAGE;
            wraw[i] = *reinterpret_cast<const moe_u32x4*>(st + gw[i] + wro[WF == 8 ? (h & 1) : 0]);
        };
        auto read_w_scale = [&](int d, int i) {
            const int dd = d < nk ? d : nk - 1;   // past the last stage: any valid byte
            wsc[i] = *reinterpret_cast<const uint16_t*>(s_lds + SCL_OFF + (wtr[i] + fr) * sp + 2 * dd);
        };
        auto dequant_w = [&](auto PAR) {
            constexpr int P = decltype(PAR)::value;   // half parity
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                if constexpr (WF == 8) {   // block 2d + P for both fragments
                    const float sc = mx_scale_operand((wsc[i] >> (8 * P)) & 0xffu);
                    fw[0][i] = mx_dequant8(wraw[i][0], wraw[i][1], sc);
                    fw[1][i] = mx_dequant8(wraw[i][2], wraw[i][3], sc);
                } else if constexpr (WF == 4) {   // block 2d + lane group
                    const float sc = mx_scale_operand((wsc[i] >> (8 * fh)) & 0xffu);
                    fw[0][i] = mx_dequant8_fp4(wraw[i][2 * P], sc);
                    fw[1][i] = mx_dequant8_fp4(wraw[i][2 * P + 1], sc);
                }
            }
        };
        // half h: multiply it from registers while reading half h+1 into the
        // same registers (each fragment right after its last MFMA of half h),
        // and, if rf, spread the loads of one refill between the MFMA groups:
        // tokens of stage `stage` (KIND 1) or weights of stage `stage` (KIND 2)
        auto half = [&](int h, auto KIND, bool rf, int stage, auto FULL) {
            constexpr int kKind = decltype(KIND)::value;
            // FULL: 1 every sub-tile live, 0 the per-MFMA test, 2 the last
            // sub-tile of the wave empty (the others live)
            constexpr int kMode = decltype(FULL)::value;
            constexpr bool kFull = kMode == 1;
            constexpr int GP = kKind == 1 ? GA : (kKind == 2 ? GW : 0);
            auto issue = [&](int q) {
                if (kKind == 1) issue_one(stage, 0, q);
                else issue_one(0, stage, GA + q);
            };
            // weight refills happen in even halves, token refills in odd ones
            constexpr int kPar = kKind == 1 ? 1 : 0;
            if (active) {
                if constexpr (MX) dequant_w(std::integral_constant<int, kPar>{});
#pragma unroll
                for (int sk = 0; sk < 2; ++sk)
#pragma unroll
                    for (int i = 0; i < NS; ++i) {
#pragma unroll
                        for (int j = 0; j < MS; ++j) {
                            if (kMode == 2 ? j < MS - 1 : (kFull || j == 0 || jlive > j))
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[sk][i], fa[sk][j], acc[i][j], 0, 0, 0);
                            if (i == NS - 1 && (kMode != 2 || j < MS - 1)) read_a(h + 1, sk, j);
                        }
                        if constexpr (!MX) {
                            read_w(h + 1, sk, i);
                        } else if (sk == 1) {   // codes (and at a new stage, scales) of half h+1
                            if (WF == 8 || kPar == 1) read_w_raw(h + 1, i);
                            if (kPar == 1) read_w_scale((h + 1) >> 1, i);
                        }
                        constexpr int SLOTS = 2 * NS;
                        const int slot = sk * NS + i;
                        if (GP > 0 && (GP >= SLOTS || (slot * GP) / SLOTS != ((slot + 1) * GP) / SLOTS)) {
#pragma unroll
                            for (int q = (slot * GP) / SLOTS; q < ((slot + 1) * GP) / SLOTS; ++q)
                                if (rf) issue(q);
                        }
                    }
            } else if (rf) {
#pragma unroll
                for (int q = 0; q < GP; ++q) issue(q);
            }
        };
        const std::integral_constant<int, 1> tokens{};
        const std::integral_constant<int, 2> weights{};

        // MX: the tile's scale rows into LDS first (the wait for stage 0 below
        // covers them): tile-row order, i.e. gated the BN/2 gate rows, then the
        // BN/2 up rows, each part a contiguous run of Ws copied in 1 KiB pieces
        if constexpr (MX) {
            const int part_bytes = (GATED ? BN / 2 : BN) * sp;   // a multiple of 1024
            const int pieces = (GATED ? 2 : 1) * (part_bytes >> 10);
            const unsigned char* s0 =
                Ws + ((size_t)e * w_rows + (GATED ? n_tile * (BN / 2) : n_tile * BN)) * sp;
            const unsigned char* s1 = Ws + ((size_t)e * w_rows + N + n_tile * (BN / 2)) * sp;
            const uint32_t ringS0 = lds_addr(s_lds + SCL_OFF);
            for (int pc = wave; pc < pieces; pc += NW) {
                const int part = (pc << 10) >= part_bytes ? 1 : 0;
                lds_dma16((part ? s1 : s0) + ((pc << 10) - part * part_bytes) + lane * 16,
                          ringS0 + (pc << 10));
            }
        }
        // prologue: the loads the k loop would have issued in earlier halves,
        // in that order (weights s in half 2(s-SW+1), tokens s in half
        // 2(s-SA)+1); then wait for stage 0
#pragma unroll
        for (int v = (2 - 2 * SW < 1 - 2 * SA ? 2 - 2 * SW : 1 - 2 * SA); v < 0; ++v) {
            if ((v & 1) == 0) {
                const int s2 = v / 2 + SW - 1;
                if (s2 >= 0 && s2 < nk)
#pragma unroll
                    for (int q = 0; q < GW; ++q) issue_one(0, s2, GA + q);
            } else {
                const int s2 = (v - 1) / 2 + SA;
                if (s2 >= 0 && s2 < nk)
#pragma unroll
                    for (int q = 0; q < GA; ++q) issue_one(s2, 0, q);
            }
        }
        if (SW - 2 < nk && SA - 1 < nk) wait_vmcnt_barrier<N_FIRST>();
        else wait_vmcnt_barrier<0>();
        if (active) {
#pragma unroll
            for (int sk = 0; sk < 2; ++sk) {
#pragma unroll
                for (int j = 0; j < MS; ++j) read_a(0, sk, j);
                if constexpr (!MX) {
#pragma unroll
                    for (int i = 0; i < NS; ++i) read_w(0, sk, i);
                }
            }
            if constexpr (MX) {
#pragma unroll
                for (int i = 0; i < NS; ++i) {
                    read_w_raw(0, i);
                    read_w_scale(0, i);
                }
            }
        }
        // Stage d: half 2d refills weights of stage d+SW-1 (slot of stage d-1,
        // whose reads were done at the barrier of half 2d-1); half 2d+1 waits
        // for stage d+1, then refills tokens of stage d+SA.
        auto k_loop = [&](auto FULL) {
            int d = 0;
            for (; d + SW < nk; ++d) {
                half(2 * d, weights, true, d + SW - 1, FULL);
                // stage d+1 landed everywhere and stage d's slots are free (see
                // above; the wave's own reads of them have returned before the
                // barrier)
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                wait_vmcnt_barrier<N_STEADY>();
                half(2 * d + 1, tokens, true, d + SA, FULL);
            }
            // last SW stages: refills only while below nk, full waits.  On the
            // last stage the read-ahead takes stale but valid LDS data that is
            // never used.
            for (; d < nk; ++d) {
                half(2 * d, weights, d + SW - 1 < nk, d + SW - 1, FULL);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                wait_vmcnt_barrier<0>();
                half(2 * d + 1, tokens, d + SA < nk, d + SA, FULL);
            }
        };
        if (!SUBSKIP || jlive >= MS) k_loop(std::integral_constant<int, 1>{});
        else if (!PROD && MS > 1 && jlive == MS - 1) k_loop(std::integral_constant<int, 2>{});
        else k_loop(std::integral_constant<int, 0>{});
        // drain the rings before the epilogue reuses them
        wait_vmcnt_barrier<0>();

        // epilogue, staged through the idle ring so that the global stores are
        // whole 16-byte pieces of contiguous output rows (written straight
        // from the MFMA layout, every store would touch 32 rows with 8 bytes
        // each).  Lane (fr, fh) holds D[n = 8p + 4fh + u][m = fr] of sub-tile
        // (i, j) in acc[i][j][4p + u] and writes those four values (8 bytes)
        // to LDS row m at pitch OP = 2*COLS + 8 bytes, so the 32 rows of one
        // write fall on 32 distinct 8-byte bank slots.
        constexpr int CPR = COLS / 8;                    // 16-byte pieces per row
        if (active) {
#pragma unroll
            for (int j = 0; j < MS; ++j) {
                unsigned char* orow = s_lds + (wm * WM + j * 32 + fr) * OP;
                if (GATED) {
#pragma unroll
                    for (int i = 0; i < NS / 2; ++i)
#pragma unroll
                        for (int p = 0; p < 4; ++p) {
                            const int col = wn * (WN / 2) + i * 32 + p * 8 + fh * 4;
                            float hv[4];
#pragma unroll
                            for (int u = 0; u < 4; ++u)
                                hv[u] = silu_f32(acc[i][j][4 * p + u]) * acc[i + NS / 2][j][4 * p + u];
                            uint2 pk;
                            pk.x = moe_f32x2_to_bf16x2(hv[0], hv[1]);
                            pk.y = moe_f32x2_to_bf16x2(hv[2], hv[3]);
                            *reinterpret_cast<uint2*>(orow + col * 2) = pk;
                        }
                } else {
#pragma unroll
                    for (int i = 0; i < NS; ++i)
#pragma unroll
                        for (int p = 0; p < 4; ++p) {
                            const int col = wn * WN + i * 32 + p * 8 + fh * 4;
                            uint2 pk;
                            pk.x = moe_f32x2_to_bf16x2(acc[i][j][4 * p], acc[i][j][4 * p + 1]);
                            pk.y = moe_f32x2_to_bf16x2(acc[i][j][4 * p + 2], acc[i][j][4 * p + 3]);
                            *reinterpret_cast<uint2*>(orow + col * 2) = pk;
                        }
                }
            }
        }
        lds_barrier();
        // Non-temporal stores: the output is read by the next kernel, not by
        // this one, so it should not displace the weight and token lines
        // that the tiles in flight share in L2, nor be left dirty there for
        // the end-of-kernel writeback.  Measured (bit-identical): static
        // capacity 5-7% faster, EP prefill at 8192 tokens 2.6-2.9%, Mixtral
        // 0.3-0.8%, the other prefill workloads 0.3-0.6%.
        uint16_t* cbase = C + (size_t)r0 * N + n_tile * COLS;
        for (int idx = tid; idx < mrows * CPR; idx += NT) {
            const int r = idx / CPR, c = idx % CPR;
            const unsigned char* src = s_lds + r * OP + c * 16;
            const uint2 lo = *reinterpret_cast<const uint2*>(src);
            const uint2 hi = *reinterpret_cast<const uint2*>(src + 8);
            const moe_u32x4 v = {lo.x, lo.y, hi.x, hi.y};
            __builtin_nontemporal_store(v, reinterpret_cast<moe_u32x4*>(cbase + (size_t)r * N + c * 8));
        }
        // every read of the staged rows is done before the ring is refilled
        lds_barrier();
    }
}

template <int BM, int BN, int WGM, int WGN, bool GATED, bool SUBSKIP, bool PACKED, bool PROD>
void launch_tiled_one(int grid, const uint16_t* A, const int32_t* row_src, int topk,
                      const int32_t* offsets, const uint16_t* W, uint16_t* C, int E, int Kd, int N,
                      int split, hipStream_t st) {
    hipLaunchKernelGGL((gemm_tiled_kernel<BM, BN, WGM, WGN, GATED, SUBSKIP, PACKED, 16, PROD>),
                       dim3(grid), dim3(64 * WGM * WGN), 0, st, A, row_src, topk, offsets, W, C, E,
                       Kd, N, split);
}

template <int BM, int BN, int WGM, int WGN, bool GATED, bool SUBSKIP = false>
hipError_t launch_tiled(int grid, const uint16_t* A, const int32_t* row_src, int topk,
                        const int32_t* offsets, const uint16_t* W, uint16_t* C, int E, int Kd,
                        int N, int split, hipStream_t st, bool packed, bool prod = false) {
    constexpr bool kProdOk = WGM * WGN == 8 && (BM / 8) % 4 == 0 && (BN / 8) % 4 == 0;
    if (prod && kProdOk) {
        if (packed)
            launch_tiled_one<BM, BN, WGM, WGN, GATED, SUBSKIP, true, kProdOk>(grid, A, row_src, topk, offsets, W, C, E, Kd, N, split, st);
        else
            launch_tiled_one<BM, BN, WGM, WGN, GATED, SUBSKIP, false, kProdOk>(grid, A, row_src, topk, offsets, W, C, E, Kd, N, split, st);
    } else if (packed) {
        launch_tiled_one<BM, BN, WGM, WGN, GATED, SUBSKIP, true, false>(grid, A, row_src, topk, offsets, W, C, E, Kd, N, split, st);
    } else {
        launch_tiled_one<BM, BN, WGM, WGN, GATED, SUBSKIP, false, false>(grid, A, row_src, topk, offsets, W, C, E, Kd, N, split, st);
    }
    return hipGetLastError();
}

template <int WF, int BM, int BN, int WGM, int WGN, bool GATED>
hipError_t launch_tiled_mx(int grid, const uint16_t* A, const int32_t* row_src, int topk,
                           const int32_t* offsets, const uint8_t* Wq, const uint8_t* Ws,
                           uint16_t* C, int E, int Kd, int N, int split, hipStream_t st,
                           bool packed) {
    // every wave fills whole weight groups (16 rows for e4m3, 32 for e2m1):
    // the plan below never asks for the shapes that cannot
    if constexpr ((BN / (WF == 8 ? 16 : 32)) % (WGM * WGN) != 0) {
        return hipErrorInvalidValue;
    } else {
        if (packed)
            hipLaunchKernelGGL((gemm_tiled_kernel<BM, BN, WGM, WGN, GATED, true, true, WF>), dim3(grid),
                               dim3(64 * WGM * WGN), 0, st, A, row_src, topk, offsets,
                               reinterpret_cast<const uint16_t*>(Wq), C, E, Kd, N, split, Ws);
        else
            hipLaunchKernelGGL((gemm_tiled_kernel<BM, BN, WGM, WGN, GATED, true, false, WF>), dim3(grid),
                               dim3(64 * WGM * WGN), 0, st, A, row_src, topk, offsets,
                               reinterpret_cast<const uint16_t*>(Wq), C, E, Kd, N, split, Ws);
        return hipGetLastError();
    }
}

template <int WF>
hipError_t launch_grouped_gemm_mx_tiled(const GemmPlan& plan, bool gated, const uint16_t* A,
                                        const int32_t* row_src, int topk, const int32_t* offsets,
                                        const uint8_t* Wq, const uint8_t* Ws, uint16_t* C, int E,
                                        int Kd, int N, hipStream_t st, bool packed) {
    const int grid = gated ? plan.grid_gateup : plan.grid_down;
    const int bn = gated ? plan.bn_gateup : plan.bn_down;
    const int split = plan.split ? 1 : 0;
#define MOE_TILED_MX(BM, BN, WGM, WGN, G) \
    launch_tiled_mx<WF, BM, BN, WGM, WGN, G>(grid, A, row_src, topk, offsets, Wq, Ws, C, E, Kd, N, split, st, packed)
    switch (plan.kind) {
        case kTiled64:
            if (gated) return MOE_TILED_MX(64, 128, 2, 2, true);
            return bn == 128 ? MOE_TILED_MX(64, 128, 2, 2, false) : MOE_TILED_MX(64, 64, 2, 2, false);
        case kTiled128:
            if (gated) return MOE_TILED_MX(128, 128, 2, 2, true);
            return bn == 128 ? MOE_TILED_MX(128, 128, 2, 2, false) : MOE_TILED_MX(128, 64, 2, 2, false);
        default:
            if (gated) return bn == 256 ? MOE_TILED_MX(192, 256, 2, 4, true) : MOE_TILED_MX(256, 128, 4, 2, true);
            if (bn == 256) return MOE_TILED_MX(192, 256, 2, 4, false);
            // 128 weight rows hold four 32-row e2m1 groups: too few for 8 waves
            if (bn == 128) return WF == 4 ? MOE_TILED_MX(128, 128, 2, 2, false)
                                          : MOE_TILED_MX(192, 128, 2, 4, false);
            return MOE_TILED_MX(128, 64, 2, 2, false);
    }
#undef MOE_TILED_MX
}

// ---------------------------------------------------------------------------
// Tiled pack layout (DeepGEMM PR #394, Summary and Motivation: weights laid
// out once in the order the kernel reads them).  The tiled kernel stages a
// weight tile as 1 KiB DMA pieces of 8 rows x 64 k-values, row r's 16-byte
// chunk c in LDS slot c ^ ring_swz(r % 32).  The pack stores, for expert e,
// 8-row group g and stage s (k-values 64s .. 64s+63), those 1 KiB
// contiguously and in slot order: piece L (0..63) = row 8g + L/8, k-values
// 64s + 8c .. +7 with c = (L % 8) ^ ring_swz((8g + L/8) % 32).  Weight tiles
// start at rows that are multiples of 32, so the swizzle a row gets in LDS is
// the one applied here.  Same size as the row-major weights.  MX codes
// (FlashInfer PR #3980, Summary: the MXFP8 backend) the same way with their
// own pieces: a stage of a row is 64 bytes of e4m3 codes (16 rows per 1 KiB,
// chunk c of row r in slot c ^ mx8_swz(r % 32)) or 32 bytes of e2m1 codes
// (32 rows, slot c ^ mx4_swz(r % 32)); the scales stay row-major.
// ---------------------------------------------------------------------------
// WF: the weight format (16 bf16, 8 e4m3 codes, 4 e2m1 codes), which sets the
// bytes of a row per stage (RBW = 128, 64, 32), the rows per 1 KiB piece
// (1024 / RBW) and the chunk swizzle the tiled kernel's DMA applies (see
// ring_swz, mx8_swz, mx4_swz); row_bytes = the bytes of one row.
template <int WF>
__global__ __launch_bounds__(256) void tiled_pack_kernel(const unsigned char* __restrict__ w,
                                                         long long pieces, int rows,
                                                         long long row_bytes,
                                                         unsigned char* __restrict__ out) {
    constexpr int RBW = WF == 16 ? 128 : (WF == 8 ? 64 : 32);
    constexpr int CH = RBW / 16;                       // 16-byte chunks of a row per stage
    constexpr int WROWS = 1024 / RBW;                  // rows per 1 KiB piece
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;   // output piece
    if (i >= pieces) return;
    const int nk = (int)(row_bytes / RBW);
    const int L = (int)(i & 63);
    const long long t = i >> 6;
    const int st = (int)(t % nk);
    const long long eg = t / nk;                       // e * (rows / WROWS) + g
    const int groups = rows / WROWS;
    const long long e = eg / groups;
    const int r = (int)(eg % groups) * WROWS + L / CH;
    const int slot = L % CH;
    const int c = WF == 16 ? slot ^ ring_swz(r & 31) : WF == 8 ? slot ^ mx8_swz(r & 31)
                                                               : slot ^ mx4_swz(r & 31);
    const unsigned char* src = w + ((size_t)e * rows + r) * (size_t)row_bytes + (size_t)st * RBW + c * 16;
    reinterpret_cast<moe_bf16x8*>(out)[i] = *reinterpret_cast<const moe_bf16x8*>(src);
}

}  // namespace

hipError_t launch_gateup_fused_dispatch(const Shape& s, const GemmPlan& plan, const uint16_t* x,
                                        const int32_t* ids, const int32_t* ntok,
                                        int32_t* offsets, int32_t* row_src, int32_t* token_row,
                                        const uint16_t* W, uint16_t* h, hipStream_t st,
                                        bool packed) {
    if (packed)
        hipLaunchKernelGGL(gemm_skinny_gateup_dispatch_kernel<true>, dim3(plan.grid_gateup),
                           dim3(256), 0, st, x, ids, ntok, s.T, s.K, s.E, offsets, row_src,
                           token_row, W, h, s.H, s.I);
    else
        hipLaunchKernelGGL(gemm_skinny_gateup_dispatch_kernel<false>, dim3(plan.grid_gateup),
                           dim3(256), 0, st, x, ids, ntok, s.T, s.K, s.E, offsets, row_src,
                           token_row, W, h, s.H, s.I);
    return hipGetLastError();
}

// Workgroups of the single-launch kernel that fit on the current device at
// once (looked up once per device): 0 if the cooperative launch cannot be
// made there.
int single_launch_grid(bool packed) {
    static std::mutex mu;
    static int cache[2][64];
    static bool have[2][64];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (!have[packed][dev]) {
        int cus = 0, coop = 0, per_cu = 0;
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        (void)hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev);
        const hipError_t e = packed
            ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, forward_tiny_single_kernel<true>, 256, 0)
            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, forward_tiny_single_kernel<false>, 256, 0);
        if (e != hipSuccess || coop == 0 || per_cu < 1 || cus < 1) per_cu = 0;
        const int grid = (per_cu > 3 ? 3 : per_cu) * cus;
        cache[packed][dev] = grid > kMaxSingleGrid ? kMaxSingleGrid : grid;
        have[packed][dev] = true;
    }
    return cache[packed][dev];
}

hipError_t launch_forward_tiny_single(const Shape& s, const uint16_t* x, const int32_t* ids,
                                      const int32_t* ntok, int32_t* offsets, int32_t* row_src,
                                      int32_t* token_row, const uint16_t* Wgu, uint16_t* h,
                                      const uint16_t* Wd, const float* w, uint16_t* out,
                                      hipStream_t st, bool packed) {
    const int grid = single_launch_grid(packed);
    if (grid <= 0) return hipErrorCooperativeLaunchTooLarge;
    if (packed)
        return launch_tiny_single<true>(s, x, ids, ntok, offsets, row_src, token_row, Wgu, h, Wd,
                                        w, out, grid, st);
    return launch_tiny_single<false>(s, x, ids, ntok, offsets, row_src, token_row, Wgu, h, Wd, w,
                                     out, grid, st);
}

hipError_t single_launch_status(unsigned int* timeouts) {
    GridSync g{};
    hipError_t e = hipMemcpyFromSymbol(&g, HIP_SYMBOL(g_grid_sync), sizeof(g), 0,
                                       hipMemcpyDeviceToHost);
    if (e != hipSuccess) return e;
    *timeouts = g.timeouts.v;
    const GridSync zero{};
    return hipMemcpyToSymbol(HIP_SYMBOL(g_grid_sync), &zero, sizeof(zero), 0, hipMemcpyHostToDevice);
}

hipError_t launch_down_combine_tiny(const Shape& s, const uint16_t* h, const int32_t* offsets,
                                    const uint16_t* W, const int32_t* token_row, const float* w,
                                    const int32_t* ntok, uint16_t* out, hipStream_t st,
                                    bool packed) {
    if (packed)
        hipLaunchKernelGGL(down_combine_tiny_kernel<true>, dim3(s.H / 16), dim3(256), 0, st, h,
                           offsets, W, s.E, s.I, s.H, token_row, w, ntok, s.T, s.K, out);
    else
        hipLaunchKernelGGL(down_combine_tiny_kernel<false>, dim3(s.H / 16), dim3(256), 0, st, h,
                           offsets, W, s.E, s.I, s.H, token_row, w, ntok, s.T, s.K, out);
    return hipGetLastError();
}

template <int FMT, bool P>
static void launch_fused_mx(const Shape& s, const uint16_t* x, const int32_t* ids,
                            const int32_t* ntok, int32_t* offsets, int32_t* row_src,
                            int32_t* token_row, const uint8_t* Wq, const uint8_t* Ws, uint16_t* h,
                            hipStream_t st) {
    if constexpr (FMT == 4) {
        if (mx_wide(FMT, s)) {
            hipLaunchKernelGGL((gemm_skinny_gateup_dispatch_mx_kernel<FMT, P, 4>),
                               dim3(mx_grid<FMT, 4>() * kNumCUs), dim3(256), 0, st, x, ids, ntok,
                               s.T, s.K, s.E, offsets, row_src, token_row, Wq, Ws, h, s.H, s.I);
            return;
        }
    }
    hipLaunchKernelGGL((gemm_skinny_gateup_dispatch_mx_kernel<FMT, P, 2>),
                       dim3(mx_grid<FMT, 2>() * kNumCUs), dim3(256), 0, st, x, ids, ntok, s.T,
                       s.K, s.E, offsets, row_src, token_row, Wq, Ws, h, s.H, s.I);
}

hipError_t launch_gateup_fused_dispatch_mx(const Shape& s, int fmt, const uint16_t* x,
                                           const int32_t* ids, const int32_t* ntok,
                                           int32_t* offsets, int32_t* row_src, int32_t* token_row,
                                           const uint8_t* Wq, const uint8_t* Ws, uint16_t* h,
                                           hipStream_t st, bool packed) {
    if (fmt == 8 && packed) launch_fused_mx<8, true>(s, x, ids, ntok, offsets, row_src, token_row, Wq, Ws, h, st);
    else if (fmt == 8) launch_fused_mx<8, false>(s, x, ids, ntok, offsets, row_src, token_row, Wq, Ws, h, st);
    else if (packed) launch_fused_mx<4, true>(s, x, ids, ntok, offsets, row_src, token_row, Wq, Ws, h, st);
    else launch_fused_mx<4, false>(s, x, ids, ntok, offsets, row_src, token_row, Wq, Ws, h, st);
    return hipGetLastError();
}

template <int FMT, bool P>
static void launch_tiny_mx(const Shape& s, const uint16_t* h, const int32_t* offsets,
                           const uint8_t* Wq, const uint8_t* Ws, const int32_t* token_row,
                           const float* w, const int32_t* ntok, uint16_t* out, hipStream_t st) {
    hipLaunchKernelGGL((down_combine_tiny_mx_kernel<FMT, P>), dim3(s.H / 16), dim3(256), 0, st, h,
                       offsets, Wq, Ws, s.E, s.I, s.H, token_row, w, ntok, s.T, s.K, out);
}

hipError_t launch_down_combine_tiny_mx(const Shape& s, int fmt, const uint16_t* h,
                                       const int32_t* offsets, const uint8_t* Wq,
                                       const uint8_t* Ws, const int32_t* token_row, const float* w,
                                       const int32_t* ntok, uint16_t* out, hipStream_t st,
                                       bool packed) {
    if (fmt == 8 && packed) launch_tiny_mx<8, true>(s, h, offsets, Wq, Ws, token_row, w, ntok, out, st);
    else if (fmt == 8) launch_tiny_mx<8, false>(s, h, offsets, Wq, Ws, token_row, w, ntok, out, st);
    else if (packed) launch_tiny_mx<4, true>(s, h, offsets, Wq, Ws, token_row, w, ntok, out, st);
    else launch_tiny_mx<4, false>(s, h, offsets, Wq, Ws, token_row, w, ntok, out, st);
    return hipGetLastError();
}

template <int FMT, bool P>
static void launch_skinny_mx(bool gated, bool wide, const uint16_t* A, const int32_t* row_src,
                             int topk, const int32_t* offsets, const uint8_t* Wq,
                             const uint8_t* Ws, uint16_t* C, int E, int Kd, int N,
                             hipStream_t st) {
    const dim3 block(256), grid2(mx_grid<FMT, 2>() * kNumCUs), grid1(mx_grid<FMT, 1>() * kNumCUs);
    if (gated) {
        if constexpr (FMT == 4) {
            if (wide) {
                hipLaunchKernelGGL((gemm_skinny_mx_kernel<FMT, true, 4, P>),
                                   dim3(mx_grid<FMT, 4>() * kNumCUs), block, 0, st, A, row_src,
                                   topk, offsets, Wq, Ws, C, E, Kd, N);
                return;
            }
        }
        hipLaunchKernelGGL((gemm_skinny_mx_kernel<FMT, true, 2, P>), grid2, block, 0, st, A,
                           row_src, topk, offsets, Wq, Ws, C, E, Kd, N);
    } else if (N % 32 == 0) {
        hipLaunchKernelGGL((gemm_skinny_mx_kernel<FMT, false, 2, P>), grid2, block, 0, st, A,
                           row_src, topk, offsets, Wq, Ws, C, E, Kd, N);
    } else {
        hipLaunchKernelGGL((gemm_skinny_mx_kernel<FMT, false, 1, P>), grid1, block, 0, st, A,
                           row_src, topk, offsets, Wq, Ws, C, E, Kd, N);
    }
}

bool mx_tiled_ok(int Kd) { return Kd % 512 == 0 && Kd / 32 <= kMxMaxKBlocks; }

hipError_t launch_grouped_gemm_mx(const Shape& s, int fmt, bool gated, const uint16_t* A,
                                  const int32_t* row_src, int topk, const int32_t* offsets,
                                  const uint8_t* Wq, const uint8_t* Ws, uint16_t* C, int Kd, int N,
                                  hipStream_t st, bool packed, int hint, bool tiled_packed) {
    // the tiled plan where the bf16 layer would take one and the tile's scales
    // fit in LDS (row-major codes, or codes in the tiled pack layout, which
    // take the tiled plan of tiled_packed_plan); else the skinny kernels
    if (tiled_packed) {   // hint: a tiled plan's kind (checked on the host)
        const GemmPlan plan = choose_plan(s, hint);
        if (packed || plan.kind == kSkinny || !mx_tiled_ok(Kd)) return hipErrorInvalidValue;
        if (fmt == 8)
            return launch_grouped_gemm_mx_tiled<8>(plan, gated, A, row_src, topk, offsets, Wq, Ws,
                                                   C, s.E, Kd, N, st, true);
        return launch_grouped_gemm_mx_tiled<4>(plan, gated, A, row_src, topk, offsets, Wq, Ws, C,
                                               s.E, Kd, N, st, true);
    }
    const GemmPlan plan = choose_plan(s, hint);
    if (!packed && plan.kind != kSkinny && mx_tiled_ok(Kd)) {
        if (fmt == 8)
            return launch_grouped_gemm_mx_tiled<8>(plan, gated, A, row_src, topk, offsets, Wq, Ws,
                                                   C, s.E, Kd, N, st, false);
        return launch_grouped_gemm_mx_tiled<4>(plan, gated, A, row_src, topk, offsets, Wq, Ws, C,
                                               s.E, Kd, N, st, false);
    }
    const bool wide = mx_wide(fmt, s);
    if (fmt == 8 && packed)
        launch_skinny_mx<8, true>(gated, wide, A, row_src, topk, offsets, Wq, Ws, C, s.E, Kd, N, st);
    else if (fmt == 8)
        launch_skinny_mx<8, false>(gated, wide, A, row_src, topk, offsets, Wq, Ws, C, s.E, Kd, N, st);
    else if (packed)
        launch_skinny_mx<4, true>(gated, wide, A, row_src, topk, offsets, Wq, Ws, C, s.E, Kd, N, st);
    else
        launch_skinny_mx<4, false>(gated, wide, A, row_src, topk, offsets, Wq, Ws, C, s.E, Kd, N, st);
    return hipGetLastError();
}

hipError_t launch_mx_quantize(int fmt, const uint16_t* w, long long nblocks, uint8_t* codes,
                              uint8_t* scales, hipStream_t st) {
    if (nblocks == 0) return hipSuccess;
    const dim3 grid((unsigned)((nblocks + 255) / 256)), block(256);
    if (fmt == 8)
        hipLaunchKernelGGL(mx_quantize_kernel<8>, grid, block, 0, st, w, nblocks, codes, scales);
    else
        hipLaunchKernelGGL(mx_quantize_kernel<4>, grid, block, 0, st, w, nblocks, codes, scales);
    return hipGetLastError();
}

hipError_t launch_mx_dequantize(int fmt, const uint8_t* codes, const uint8_t* scales,
                                long long nblocks, uint16_t* w, hipStream_t st) {
    if (nblocks == 0) return hipSuccess;
    const dim3 grid((unsigned)((nblocks + 255) / 256)), block(256);
    if (fmt == 8)
        hipLaunchKernelGGL(mx_dequantize_kernel<8>, grid, block, 0, st, codes, scales, nblocks, w);
    else
        hipLaunchKernelGGL(mx_dequantize_kernel<4>, grid, block, 0, st, codes, scales, nblocks, w);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm_packed(const Shape& s, bool gated, const uint16_t* A,
                                      const int32_t* row_src, int topk, const int32_t* offsets,
                                      const uint16_t* W, uint16_t* C, int Kd, int N,
                                      hipStream_t st) {
    const dim3 grid(4 * kNumCUs), block(256);
    if (gated)
        hipLaunchKernelGGL((gemm_skinny_kernel<true, 1, true>), grid, block, 0, st, A, row_src,
                           topk, offsets, W, C, s.E, Kd, N);
    else if (N % 32 == 0)
        hipLaunchKernelGGL((gemm_skinny_kernel<false, 2, true>), grid, block, 0, st, A, row_src,
                           topk, offsets, W, C, s.E, Kd, N);
    else
        hipLaunchKernelGGL((gemm_skinny_kernel<false, 1, true>), grid, block, 0, st, A, row_src,
                           topk, offsets, W, C, s.E, Kd, N);
    return hipGetLastError();
}

hipError_t launch_tiled_pack(const uint16_t* w, int experts, int rows, int Kd, uint16_t* out,
                             hipStream_t st) {
    const long long pieces = (long long)experts * rows * (Kd / 8);
    if (pieces == 0) return hipSuccess;
    hipLaunchKernelGGL(tiled_pack_kernel<16>, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0,
                       st, reinterpret_cast<const unsigned char*>(w), pieces, rows,
                       (long long)Kd * 2, reinterpret_cast<unsigned char*>(out));
    return hipGetLastError();
}

hipError_t launch_mx_tiled_pack(int fmt, const uint8_t* codes, int experts, int rows, int Kd,
                                uint8_t* out, hipStream_t st) {
    const long long row_bytes = (long long)Kd * fmt / 8;
    const long long pieces = (long long)experts * rows * (row_bytes / 16);
    if (pieces == 0) return hipSuccess;
    const dim3 grid((unsigned)((pieces + 255) / 256)), block(256);
    if (fmt == 8)
        hipLaunchKernelGGL(tiled_pack_kernel<8>, grid, block, 0, st, codes, pieces, rows, row_bytes,
                           out);
    else
        hipLaunchKernelGGL(tiled_pack_kernel<4>, grid, block, 0, st, codes, pieces, rows, row_bytes,
                           out);
    return hipGetLastError();
}

hipError_t launch_skinny_pack(const uint16_t* w, int experts, int rows, int Kd, bool gated,
                              uint16_t* out, hipStream_t st) {
    const long long pieces = (long long)experts * rows * (Kd / 8);
    if (pieces == 0) return hipSuccess;
    hipLaunchKernelGGL(skinny_pack_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0,
                       st, w, pieces, rows, Kd, gated ? 1 : 0, out);
    return hipGetLastError();
}

GemmPlan choose_plan(const Shape& s, int hint) {
    GemmPlan p{};
    int kind = hint;
    const double rows_per_expert = (double)s.T * s.K / (double)s.E;
    if (kind < kSkinny || kind > kTiledLarge) {
        kind = rows_per_expert <= 24.0 ? kSkinny
             : rows_per_expert <= 96.0 ? kTiled64 : kTiledLarge;
    }
    p.kind = kind;
    p.split = s.E >= 32;   // tiled kinds: two halves of the tile list in flight
    if (kind == kSkinny) {
        p.grid_gateup = p.grid_down = 4 * kNumCUs;   // 4 workgroups fit per CU
        p.bn_gateup = p.bn_down = 16;
    } else if (kind == kTiledLarge) {
        // 192 token rows per tile.  gate-up: 128 gate + 128 up rows (256-row
        // token tiles with 64 + 64 when I is not a multiple of 128); down: 256
        // or 128 weight rows, whichever fills the last round of tiles better
        p.bn_gateup = (s.I % 128 == 0) ? 256 : 128;
        p.bn_down = (s.H % 128 == 0) ? 128 : 64;
        if (s.H % 256 == 0) {
            const double m_tiles = s.E * std::ceil((double)s.T * s.K / s.E / 192.0);
            auto fill = [&](int bn) {
                const double t = m_tiles * (s.H / bn);
                return t / (std::ceil(t / kNumCUs) * kNumCUs);
            };
            if (fill(256) >= 0.9 * fill(128)) p.bn_down = 256;
        }
        p.grid_gateup = p.grid_down = kNumCUs;
        // Tiles that hold few token rows: a large part of each stage's MFMA
        // work sits in waves 0-3, and with all eight waves issuing DMAs the
        // two waves of a SIMD tend to stall on the address unit at the same
        // points.  Letting waves 0-3 issue every DMA leaves waves 4-7 free to
        // keep the matrix pipes busy.  Measured (outputs bit-identical): EP
        // prefill at 8192 tokens 6% faster, Zipf-routed 4-6%, static
        // capacity 2%; at ~1024 rows per expert (Mixtral) 3% slower, so only
        // below the threshold the sub-tile skipping is tuned for.
        p.prod = rows_per_expert < 768.0;
    } else {
        p.bn_gateup = 128;                          // 64 gate + 64 up rows
        p.bn_down = (s.H % 128 == 0) ? 128 : 64;
        p.grid_gateup = p.grid_down = 2 * kNumCUs;
    }
    return p;
}

hipError_t launch_grouped_gemm(const Shape& s, const GemmPlan& plan, bool gated,
                               const uint16_t* A, const int32_t* row_src, int topk,
                               const int32_t* offsets, const uint16_t* W, uint16_t* C, int Kd,
                               int N, hipStream_t st, bool tiled_packed) {
    const int grid = gated ? plan.grid_gateup : plan.grid_down;
    const int bn = gated ? plan.bn_gateup : plan.bn_down;
    const int split = plan.split ? 1 : 0;
#define MOE_TILED(BM, BN, WGM, WGN, G) \
    launch_tiled<BM, BN, WGM, WGN, G>(grid, A, row_src, topk, offsets, W, C, s.E, Kd, N, split, st, tiled_packed)
#define MOE_TILED_S(BM, BN, WGM, WGN, G) \
    launch_tiled<BM, BN, WGM, WGN, G, true>(grid, A, row_src, topk, offsets, W, C, s.E, Kd, N, split, st, tiled_packed, plan.prod)
    if (tiled_packed && plan.kind == kSkinny) return hipErrorInvalidValue;   // checked on the host
    switch (plan.kind) {
        case kSkinny:
            if (gated)
                hipLaunchKernelGGL((gemm_skinny_kernel<true, 1>), dim3(grid), dim3(256), 0, st, A,
                                   row_src, topk, offsets, W, C, s.E, Kd, N);
            else if (N % 32 == 0)
                hipLaunchKernelGGL((gemm_skinny_kernel<false, 2>), dim3(grid), dim3(256), 0, st, A,
                                   row_src, topk, offsets, W, C, s.E, Kd, N);
            else
                hipLaunchKernelGGL((gemm_skinny_kernel<false, 1>), dim3(grid), dim3(256), 0, st, A,
                                   row_src, topk, offsets, W, C, s.E, Kd, N);
            return hipGetLastError();
        case kTiled64:
            if (gated) return MOE_TILED(64, 128, 2, 2, true);
            return bn == 128 ? MOE_TILED(64, 128, 2, 2, false) : MOE_TILED(64, 64, 2, 2, false);
        case kTiled128:
            if (gated) return MOE_TILED(128, 128, 2, 2, true);
            return bn == 128 ? MOE_TILED(128, 128, 2, 2, false) : MOE_TILED(128, 64, 2, 2, false);
        default:
            // 192 = 2 x 96 token rows: a wave holds 3 x 2 sub-tiles of 32 x 32.
            // Sub-tiles past the valid rows skip their MFMAs (SUBSKIP); waves
            // whose sub-tiles all hold rows run a k loop without that test.
            if (gated) return bn == 256 ? MOE_TILED_S(192, 256, 2, 4, true) : MOE_TILED_S(256, 128, 4, 2, true);
            return bn == 256 ? MOE_TILED_S(192, 256, 2, 4, false)
                 : bn == 128 ? MOE_TILED_S(192, 128, 2, 4, false) : MOE_TILED(128, 64, 2, 2, false);
    }
#undef MOE_TILED
#undef MOE_TILED_S
}

}  // namespace moe
