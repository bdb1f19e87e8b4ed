// Grouped BF16 GEMMs of the dispatched-expert MLP on gfx950 MFMA (TileOps PR
// #1738 "[Refactor][MoE] Separate dispatched expert compute", Review
// follow-up: a gate-up grouped GEMM whose epilogue applies the gated
// pointwise op, then a down grouped GEMM; one column mapping and one
// epilogue serve every row policy).
//
// Both kernels are persistent and fixed-grid.  Each workgroup first turns the
// GPU-resident expert_offsets into an LDS table of per-expert tile starts
// (tiles = ceil(M_e / BM) * n_tiles), so the valid-row count bounds all the
// work on the device and the same launch serves every T_v (graph replay).
// Tiles of one expert are numbered m-fastest, so the m-tiles that reuse one
// weight tile run at the same time and share it through L2 / MALL.
//
// MFMA operands are "swapped": the weight rows are the A operand (MFMA rows)
// and the dispatched token rows the B operand (MFMA columns), so an
// accumulator lane holds 4 consecutive output columns of one token row.
// v_mfma_f32_16x16x32_bf16 lane layout (gfx950): lane l supplies A row l%16
// and B column l%16 with 8 k-values each; lane groups l/16 = 0..3 cover k
// blocks of 8; D[4*(l/16)+i][l%16] lands in accumulator i.
//
// gated: W = [E, 2N, Kd] (rows [0,N) gate, [N,2N) up), C = bf16(silu(g)*u) [cap, N]
// plain: W = [E, N, Kd],                                 C = bf16(acc)      [cap, N]
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ moe_bf16x8 load16(const uint16_t* p) {
    return *reinterpret_cast<const moe_bf16x8*>(p);
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

// Tile table: s_start[e] = sum_{e' < e} ceil(M_e'/BM) * n_tiles, s_start[E] = total.
template <int BM>
__device__ __forceinline__ int build_tile_table(const int32_t* __restrict__ offsets, int E,
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
// Tile = 16 weight rows x 16 token rows x the whole K, split over the 4 waves
// of the workgroup (contiguous k ranges), reduced through LDS in wave order.
// gated: the 16 weight rows are 8 gate rows and the 8 matching up rows, so a
// tile produces 8 output columns; plain: 16 output columns.
// ---------------------------------------------------------------------------
template <bool GATED>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ row_src, int topk,
    const int32_t* __restrict__ offsets, const uint16_t* __restrict__ W,
    uint16_t* __restrict__ C, int E, int Kd, int N) {
    constexpr int BM = 16;
    constexpr int COLS = GATED ? 8 : 16;
    __shared__ int s_start[kMaxExperts + 1];
    __shared__ int s_wave[4];
    __shared__ float s_red[4][16][17];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int n_tiles = N / COLS;
    const int w_rows = GATED ? 2 * N : N;
    const int total = build_tile_table<BM>(offsets, E, n_tiles, s_start, s_wave);

    const int ksteps = Kd / 32;
    const int ks0 = (wave * ksteps) / 4, ks1 = ((wave + 1) * ksteps) / 4;

    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const int e = find_expert(s_start, E, tile);
        const int row0 = offsets[e];
        const int me = offsets[e + 1] - row0;
        const int mt = (me + BM - 1) / BM;
        const int local = tile - s_start[e];
        const int m_tile = local % mt, n_tile = local / mt;
        const int r0 = row0 + m_tile * BM;
        const int mrows = (me - m_tile * BM) < BM ? (me - m_tile * BM) : BM;

        int wrow;
        if (GATED) wrow = (li < 8) ? (n_tile * 8 + li) : (N + n_tile * 8 + (li - 8));
        else wrow = n_tile * 16 + li;
        const uint16_t* wp = W + ((size_t)e * w_rows + wrow) * (size_t)Kd + lg * 8;
        const bool mvalid = li < mrows;
        const int rr = r0 + (mvalid ? li : 0);
        const long long arow = row_src ? (long long)(row_src[rr] / topk) : (long long)rr;
        const uint16_t* ap = A + (size_t)arow * Kd + lg * 8;

        moe_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const moe_bf16x8 zero = {};
        int ks = ks0;
        for (; ks + 8 <= ks1; ks += 8) {
            moe_bf16x8 wv[8], av[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) wv[u] = load16(wp + (size_t)(ks + u) * 32);
#pragma unroll
            for (int u = 0; u < 8; ++u) av[u] = mvalid ? load16(ap + (size_t)(ks + u) * 32) : zero;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[u], av[u], acc, 0, 0, 0);
        }
        for (; ks < ks1; ++ks) {
            const moe_bf16x8 wv = load16(wp + (size_t)ks * 32);
            const moe_bf16x8 av = mvalid ? load16(ap + (size_t)ks * 32) : zero;
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv, av, acc, 0, 0, 0);
        }

#pragma unroll
        for (int i = 0; i < 4; ++i) s_red[wave][4 * lg + i][li] = acc[i];
        __syncthreads();
        if (GATED) {
            if (tid < 128) {
                const int m = tid >> 3, c = tid & 7;
                if (m < mrows) {
                    float g = 0.f, u = 0.f;
#pragma unroll
                    for (int w = 0; w < 4; ++w) { g += s_red[w][c][m]; u += s_red[w][8 + c][m]; }
                    C[(size_t)(r0 + m) * N + n_tile * 8 + c] = moe_f32_to_bf16(silu_f32(g) * u);
                }
            }
        } else {
            const int m = tid >> 4, c = tid & 15;
            if (m < mrows) {
                float y = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) y += s_red[w][c][m];
                C[(size_t)(r0 + m) * N + n_tile * 16 + c] = moe_f32_to_bf16(y);
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Tiled kernel: BM token rows x BN weight rows per tile, BK = 64, operands
// staged through double-buffered LDS (row pitch 72 bf16 = 144 B, so the 8
// lanes of one 128-byte LDS access phase start 16 B apart in bank space).
// 4 waves in a 2 (weight) x 2 (token) grid; each wave owns (BN/2) x (BM/2)
// of the tile as 16x16 MFMA sub-tiles.  gated: tile rows [0, BN/2) are gate
// columns n0.. and [BN/2, BN) the matching up columns, and each wave takes
// the same column range from both halves so gate and up of one output meet
// in one lane.
// ---------------------------------------------------------------------------
constexpr int kBK = 64;
constexpr int kPitch = 72;

template <int BM, int BN, bool GATED>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ row_src, int topk,
    const int32_t* __restrict__ offsets, const uint16_t* __restrict__ W,
    uint16_t* __restrict__ C, int E, int Kd, int N) {
    static_assert(BM % 32 == 0 && BN % 64 == 0, "tile shape");
    constexpr int WN = BN / 2, WM = BM / 2;          // per-wave extent
    constexpr int NS = WN / 16, MS = WM / 16;        // 16x16 sub-tiles per wave
    constexpr int COLS = GATED ? BN / 2 : BN;        // output columns per tile
    constexpr int WPASS = BN / 32, APASS = BM / 32;  // 16-B loads per thread per k-step

    __shared__ int s_start[kMaxExperts + 1];
    __shared__ int s_wave[4];
    __shared__ __attribute__((aligned(16))) uint16_t s_w[2][BN * kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t s_a[2][BM * kPitch];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int wn = wave >> 1, wm = wave & 1;
    const int n_tiles = N / COLS;
    const int w_rows = GATED ? 2 * N : N;
    const int total = build_tile_table<BM>(offsets, E, n_tiles, s_start, s_wave);
    const int nk = Kd / kBK;

    // XCD-aware order: workgroup b runs on XCD b % 8; give each XCD a
    // contiguous run of logical tiles so neighbouring m-tiles share its L2.
    const int G = gridDim.x;
    const int lb = (G % 8 == 0) ? ((int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8))
                                : (int)blockIdx.x;

    // global -> LDS copy roles: 8 threads per 128-byte row segment
    const int cp_row = tid >> 3, cp_col = (tid & 7) * 8;

    for (int tile = lb; tile < total; tile += G) {
        const int e = find_expert(s_start, E, tile);
        const int row0 = offsets[e];
        const int me = offsets[e + 1] - row0;
        const int mt = (me + BM - 1) / BM;
        const int local = tile - s_start[e];
        const int m_tile = local % mt, n_tile = local / mt;
        const int r0 = row0 + m_tile * BM;
        const int mrows = (me - m_tile * BM) < BM ? (me - m_tile * BM) : BM;

        const uint16_t* wsrc[WPASS];
#pragma unroll
        for (int p = 0; p < WPASS; ++p) {
            const int tr = cp_row + 32 * p;
            int wr;
            if (GATED) wr = (tr < BN / 2) ? (n_tile * (BN / 2) + tr) : (N + n_tile * (BN / 2) + tr - BN / 2);
            else wr = n_tile * BN + tr;
            wsrc[p] = W + ((size_t)e * w_rows + wr) * (size_t)Kd + cp_col;
        }
        const uint16_t* asrc[APASS];
#pragma unroll
        for (int p = 0; p < APASS; ++p) {
            const int tr = cp_row + 32 * p;
            const int rr = r0 + (tr < mrows ? tr : mrows - 1);
            const long long arow = row_src ? (long long)(row_src[rr] / topk) : (long long)rr;
            asrc[p] = A + (size_t)arow * Kd + cp_col;
        }

        moe_f32x4 acc[NS][MS];
#pragma unroll
        for (int i = 0; i < NS; ++i)
#pragma unroll
            for (int j = 0; j < MS; ++j) acc[i][j] = (moe_f32x4){0.f, 0.f, 0.f, 0.f};

        {
            uint4 rw[WPASS], ra[APASS];
#pragma unroll
            for (int p = 0; p < WPASS; ++p) rw[p] = *reinterpret_cast<const uint4*>(wsrc[p]);
#pragma unroll
            for (int p = 0; p < APASS; ++p) ra[p] = *reinterpret_cast<const uint4*>(asrc[p]);
#pragma unroll
            for (int p = 0; p < WPASS; ++p)
                *reinterpret_cast<uint4*>(&s_w[0][(cp_row + 32 * p) * kPitch + cp_col]) = rw[p];
#pragma unroll
            for (int p = 0; p < APASS; ++p)
                *reinterpret_cast<uint4*>(&s_a[0][(cp_row + 32 * p) * kPitch + cp_col]) = ra[p];
        }
        __syncthreads();

        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            // Prefetch the next k-step (the last iteration re-reads its own
            // step, which lands in the idle buffer and is never consumed).
            const size_t ko = (size_t)(kt + 1 < nk ? kt + 1 : kt) * kBK;
            uint4 rw[WPASS], ra[APASS];
#pragma unroll
            for (int p = 0; p < WPASS; ++p) rw[p] = *reinterpret_cast<const uint4*>(wsrc[p] + ko);
#pragma unroll
            for (int p = 0; p < APASS; ++p) ra[p] = *reinterpret_cast<const uint4*>(asrc[p] + ko);
#pragma unroll
            for (int kk = 0; kk < kBK / 32; ++kk) {
                moe_bf16x8 fw[NS], fa[MS];
#pragma unroll
                for (int i = 0; i < NS; ++i) {
                    int trow;
                    if (GATED) trow = (i < NS / 2) ? (wn * (WN / 2) + i * 16 + li)
                                                   : (BN / 2 + wn * (WN / 2) + (i - NS / 2) * 16 + li);
                    else trow = wn * WN + i * 16 + li;
                    fw[i] = *reinterpret_cast<const moe_bf16x8*>(&s_w[cur][trow * kPitch + kk * 32 + lg * 8]);
                }
#pragma unroll
                for (int j = 0; j < MS; ++j) {
                    const int arow = wm * WM + j * 16 + li;
                    fa[j] = *reinterpret_cast<const moe_bf16x8*>(&s_a[cur][arow * kPitch + kk * 32 + lg * 8]);
                }
#pragma unroll
                for (int i = 0; i < NS; ++i)
#pragma unroll
                    for (int j = 0; j < MS; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[i], fa[j], acc[i][j], 0, 0, 0);
            }
#pragma unroll
            for (int p = 0; p < WPASS; ++p)
                *reinterpret_cast<uint4*>(&s_w[cur ^ 1][(cp_row + 32 * p) * kPitch + cp_col]) = rw[p];
#pragma unroll
            for (int p = 0; p < APASS; ++p)
                *reinterpret_cast<uint4*>(&s_a[cur ^ 1][(cp_row + 32 * p) * kPitch + cp_col]) = ra[p];
            __syncthreads();
        }

        // epilogue: lane holds D[n = 16*i + 4*lg + q][m = 16*j + li], q = 0..3
#pragma unroll
        for (int j = 0; j < MS; ++j) {
            const int m = wm * WM + j * 16 + li;
            if (m >= mrows) continue;
            uint16_t* crow = C + (size_t)(r0 + m) * N;
            if (GATED) {
#pragma unroll
                for (int i = 0; i < NS / 2; ++i) {
                    const int col = n_tile * COLS + wn * (WN / 2) + i * 16 + lg * 4;
                    uint16_t hv[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        hv[q] = moe_f32_to_bf16(silu_f32(acc[i][j][q]) * acc[i + NS / 2][j][q]);
                    uint2 pk;
                    pk.x = (uint32_t)hv[0] | ((uint32_t)hv[1] << 16);
                    pk.y = (uint32_t)hv[2] | ((uint32_t)hv[3] << 16);
                    *reinterpret_cast<uint2*>(crow + col) = pk;
                }
            } else {
#pragma unroll
                for (int i = 0; i < NS; ++i) {
                    const int col = n_tile * COLS + wn * WN + i * 16 + lg * 4;
                    uint2 pk;
                    pk.x = (uint32_t)moe_f32_to_bf16(acc[i][j][0]) | ((uint32_t)moe_f32_to_bf16(acc[i][j][1]) << 16);
                    pk.y = (uint32_t)moe_f32_to_bf16(acc[i][j][2]) | ((uint32_t)moe_f32_to_bf16(acc[i][j][3]) << 16);
                    *reinterpret_cast<uint2*>(crow + col) = pk;
                }
            }
        }
    }
}

template <int BM, int BN, bool GATED>
hipError_t launch_tiled(int grid, const uint16_t* A, const int32_t* row_src, int topk,
                        const int32_t* offsets, const uint16_t* W, uint16_t* C, int E, int Kd,
                        int N, hipStream_t st) {
    hipLaunchKernelGGL((gemm_tiled_kernel<BM, BN, GATED>), dim3(grid), dim3(256), 0, st, A,
                       row_src, topk, offsets, W, C, E, Kd, N);
    return hipGetLastError();
}

}  // namespace

GemmPlan choose_plan(const Shape& s, int hint) {
    GemmPlan p{};
    int kind = hint;
    if (kind < kSkinny || kind > kTiled128) {
        const double rows_per_expert = (double)s.T * s.K / (double)s.E;
        kind = rows_per_expert <= 24.0 ? kSkinny : (rows_per_expert <= 96.0 ? kTiled64 : kTiled128);
    }
    p.kind = kind;
    if (kind == kSkinny) {
        p.grid_gateup = p.grid_down = 4 * kNumCUs;
        p.bn_gateup = p.bn_down = 16;
    } else {
        p.bn_gateup = (s.I % 64 == 0) ? 128 : 64;   // 64 gate + 64 up rows
        p.bn_down = (s.H % 128 == 0) ? 128 : 64;
        p.grid_gateup = p.grid_down = 2 * kNumCUs;
    }
    return p;
}

hipError_t launch_grouped_gemm(const Shape& s, const GemmPlan& plan, bool gated,
                               const uint16_t* A, const int32_t* row_src, int topk,
                               const int32_t* offsets, const uint16_t* W, uint16_t* C, int Kd,
                               int N, hipStream_t st) {
    const int grid = gated ? plan.grid_gateup : plan.grid_down;
    if (plan.kind == kSkinny) {
        if (gated)
            hipLaunchKernelGGL(gemm_skinny_kernel<true>, dim3(grid), dim3(256), 0, st, A, row_src,
                               topk, offsets, W, C, s.E, Kd, N);
        else
            hipLaunchKernelGGL(gemm_skinny_kernel<false>, dim3(grid), dim3(256), 0, st, A, row_src,
                               topk, offsets, W, C, s.E, Kd, N);
        return hipGetLastError();
    }
    const int bn = gated ? plan.bn_gateup : plan.bn_down;
    if (plan.kind == kTiled64) {
        if (gated) return bn == 128 ? launch_tiled<64, 128, true>(grid, A, row_src, topk, offsets, W, C, s.E, Kd, N, st)
                                    : launch_tiled<64, 64, true>(grid, A, row_src, topk, offsets, W, C, s.E, Kd, N, st);
        return bn == 128 ? launch_tiled<64, 128, false>(grid, A, row_src, topk, offsets, W, C, s.E, Kd, N, st)
                         : launch_tiled<64, 64, false>(grid, A, row_src, topk, offsets, W, C, s.E, Kd, N, st);
    }
    if (gated) return bn == 128 ? launch_tiled<128, 128, true>(grid, A, row_src, topk, offsets, W, C, s.E, Kd, N, st)
                                : launch_tiled<128, 64, true>(grid, A, row_src, topk, offsets, W, C, s.E, Kd, N, st);
    return bn == 128 ? launch_tiled<128, 128, false>(grid, A, row_src, topk, offsets, W, C, s.E, Kd, N, st)
                     : launch_tiled<128, 64, false>(grid, A, row_src, topk, offsets, W, C, s.E, Kd, N, st);
}

}  // namespace moe
