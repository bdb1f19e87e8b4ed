// Internal declarations shared by the kernels and the host entry points of
// libmoe_mi355x.so (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxExperts = 512;
constexpr int kDispatchThreads = 1024;
constexpr int kDispatchChunk = 4096;     // assignments per block, multi-block dispatch
constexpr int kDispatchSingleMax = 8192; // up to this many assignments: one block does it all
constexpr int kNumCUs = 256;
constexpr int kFusedDispatchMax = 1024;  // T*K up to this: the skinny gate-up kernel dispatches

struct Shape {
    int T, K, E, H, I, cap;
};

// Grouped-GEMM plan, chosen on the host from host-known sizes only.
enum GemmKind { kSkinny = 1, kTiled64 = 2, kTiled128 = 3, kTiledLarge = 4 };
struct GemmPlan {
    int kind;
    int grid_gateup, grid_down;
    int bn_gateup, bn_down;  // weight rows per tile (tiled kinds)
    bool split;              // tiled: XCDs 0-3 and 4-7 walk the two halves of the tile list
    bool prod;               // large tiles: waves 0-3 issue every DMA of the rings
};

GemmPlan choose_plan(const Shape& s, int hint);

inline int dispatch_blocks(const Shape& s) {
    long long n = (long long)s.T * s.K;
    if (n <= kDispatchSingleMax) return 1;
    return (int)((n + kDispatchChunk - 1) / kDispatchChunk);
}

// The router fused into dispatch: up to kRouteSingleMax assignments one
// block routes and dispatches; above it the routing is done by a counting
// grid over chunks of kDispatchChunk / ratio assignments (ratio 4 when K <= 4,
// so that no thread routes more than one token), with route_count_rows(s)
// histogram rows, then scanned and scattered as in the multi-block dispatch.
constexpr int kRouteSingleMax = 1024;
inline int route_count_ratio(int K) { return K <= 4 ? 4 : 1; }
inline int route_count_rows(const Shape& s) {
    const long long n = (long long)s.T * s.K;
    if (n <= kRouteSingleMax) return 0;
    const long long chunk = kDispatchChunk / route_count_ratio(s.K);
    return (int)((n + chunk - 1) / chunk);
}

// ---- launches (each returns hipGetLastError() of its launches) ----------
hipError_t launch_dispatch(const Shape& s, const int32_t* ids, const int32_t* ntok,
                           int32_t* offsets, int32_t* row_src, int32_t* token_row,
                           int32_t* blk_counts, hipStream_t st);
// The router step fused ahead of dispatch: ids [T,K] and weights [T,K] (rows
// t < T_v) from fp32 logits [T,G] (G >= 1 router experts; ids >= E are
// dropped by the dispatch like any non-local id), then the dispatch on them.
hipError_t launch_router_dispatch(const Shape& s, const float* logits, int G, const int32_t* ntok,
                                  int32_t* ids, float* wts, int32_t* offsets, int32_t* row_src,
                                  int32_t* token_row, int32_t* blk_counts, hipStream_t st);
hipError_t launch_gather(const Shape& s, const uint16_t* x, const int32_t* offsets,
                         const int32_t* row_src, uint16_t* x_disp, hipStream_t st);
// C[r, :] for the dispatched rows r < R:
//   gated: C = bf16(silu(A W_gate^T) * (A W_up^T)), W = [E, 2N, Kd], C: [cap, N]
//   plain: C = bf16(A W^T),                            W = [E, N, Kd],  C: [cap, N]
// A row of dispatched row r is A[row_src ? row_src[r] / topk : r].
// tiled_packed: W is in the tiled pack layout (launch_tiled_pack); the plan
// must be a tiled one.
hipError_t launch_grouped_gemm(const Shape& s, const GemmPlan& plan, bool gated,
                               const uint16_t* A, const int32_t* row_src, int topk,
                               const int32_t* offsets, const uint16_t* W, uint16_t* C,
                               int Kd, int N, hipStream_t st, bool tiled_packed = false);
// bf16 weights [experts, rows, Kd] (rows % 32 == 0, Kd % 64 == 0) -> tiled pack
// layout: per expert, 8-row group and 64-value stage, the 1 KiB the tiled
// kernel's DMA instruction stages, contiguous and in LDS slot order.
hipError_t launch_tiled_pack(const uint16_t* w, int experts, int rows, int Kd, uint16_t* out,
                             hipStream_t st);
// Gate-up GEMM of the skinny plan with the local dispatch done inside: every
// workgroup builds the dispatch of the T*K (<= kFusedDispatchMax) assignments
// in LDS; workgroup 0 also writes expert_offsets, row_src and token_row.
hipError_t launch_gateup_fused_dispatch(const Shape& s, const GemmPlan& plan, const uint16_t* x,
                                        const int32_t* ids, const int32_t* ntok,
                                        int32_t* offsets, int32_t* row_src, int32_t* token_row,
                                        const uint16_t* W, uint16_t* h, hipStream_t st,
                                        bool packed = false);
// Down GEMM + weighted combine in one launch for tiny batches: usable when
// T*K <= kTinyRows and I % 1024 == 0 (tiny_down_ok); needs the expert_offsets
// and token_row of the fused gate-up kernel.
constexpr int kTinyRows = 8;
inline bool tiny_down_ok(const Shape& s) {
    return (long long)s.T * s.K <= kTinyRows && s.I % 1024 == 0 && s.H % 16 == 0;
}
// The tiny-batch layer (tiny_down_ok, T*K <= kTinyRows) in one cooperative
// launch: dispatch + gate-up, a grid barrier, down + combine.  Returns
// hipErrorCooperativeLaunchTooLarge when the device cannot hold the grid.
hipError_t launch_forward_tiny_single(const Shape& s, const uint16_t* x, const int32_t* ids,
                                      const int32_t* ntok, int32_t* offsets, int32_t* row_src,
                                      int32_t* token_row, const uint16_t* Wgu, uint16_t* h,
                                      const uint16_t* Wd, const float* w, uint16_t* out,
                                      hipStream_t st, bool packed = false);
// Barrier timeouts recorded by single launches on the current device since
// the last call (host synchronous; resets the barrier state).
hipError_t single_launch_status(unsigned int* timeouts);
hipError_t launch_down_combine_tiny(const Shape& s, const uint16_t* h, const int32_t* offsets,
                                    const uint16_t* W, const int32_t* token_row, const float* w,
                                    const int32_t* ntok, uint16_t* out, hipStream_t st,
                                    bool packed = false);
// The skinny kernels on weights in the skinny pack layout (grid 4 x CUs).
hipError_t launch_grouped_gemm_packed(const Shape& s, bool gated, const uint16_t* A,
                                      const int32_t* row_src, int topk, const int32_t* offsets,
                                      const uint16_t* W, uint16_t* C, int Kd, int N,
                                      hipStream_t st);
// bf16 weights [experts, rows, Kd] -> skinny pack layout (rows % 16 == 0; gated:
// W_gateup with gate rows [0, rows/2) and up rows [rows/2, rows)).
hipError_t launch_skinny_pack(const uint16_t* w, int experts, int rows, int Kd, bool gated,
                              uint16_t* out, hipStream_t st);
// ---- MX weights: fmt 8 = MXFP8 (e4m3 codes, one byte per value), fmt 4 =
// MXFP4 (e2m1 codes, two per byte, low nibble first); codes uint8 [.., rows,
// Kd * fmt / 8], scales uint8 [.., rows, Kd/32] (e8m0, one per 32 values).
// The skinny kernels on MX weights (grid 3 x CUs), same contracts as above;
// MXFP4 needs Kd % 128 == 0 (checked on the host).  packed: the codes are in
// the skinny pack layout (launch_skinny_pack on the codes viewed as 16-bit
// values, k = code bytes per row / 2); the scales stay row-major.
hipError_t launch_gateup_fused_dispatch_mx(const Shape& s, int fmt, const uint16_t* x,
                                           const int32_t* ids, const int32_t* ntok,
                                           int32_t* offsets, int32_t* row_src, int32_t* token_row,
                                           const uint8_t* Wq, const uint8_t* Ws, uint16_t* h,
                                           hipStream_t st, bool packed = false);
hipError_t launch_down_combine_tiny_mx(const Shape& s, int fmt, const uint16_t* h,
                                       const int32_t* offsets, const uint8_t* Wq,
                                       const uint8_t* Ws, const int32_t* token_row, const float* w,
                                       const int32_t* ntok, uint16_t* out, hipStream_t st,
                                       bool packed = false);
// The grouped GEMM on MX weights: the tiled plan (MFMA tiles of the bf16
// plan, codes staged through LDS and dequantized on the fragment reads, the
// tile's scales in LDS) when choose_plan(s, hint) is a tiled one, the codes
// are row-major and mx_tiled_ok(Kd); else the skinny MX kernels (packed:
// codes in the skinny pack layout).  tiled_packed: codes in the tiled pack
// layout (launch_mx_tiled_pack); hint must then name a tiled plan and
// mx_tiled_ok(Kd) hold.
bool mx_tiled_ok(int Kd);
hipError_t launch_grouped_gemm_mx(const Shape& s, int fmt, bool gated, const uint16_t* A,
                                  const int32_t* row_src, int topk, const int32_t* offsets,
                                  const uint8_t* Wq, const uint8_t* Ws, uint16_t* C, int Kd, int N,
                                  hipStream_t st, bool packed = false, int hint = 0,
                                  bool tiled_packed = false);
// MX codes [experts, rows, Kd * fmt / 8 bytes] (rows % 32 == 0, Kd % 64 == 0)
// -> the tiled pack layout of those codes (1 KiB DMA pieces of 16 rows x 64
// bytes for e4m3, 32 rows x 32 bytes for e2m1, contiguous, in slot order).
hipError_t launch_mx_tiled_pack(int fmt, const uint8_t* codes, int experts, int rows, int Kd,
                                uint8_t* out, hipStream_t st);
// nblocks blocks of 32 consecutive bf16 values <-> 32 codes + 1 scale each
hipError_t launch_mx_quantize(int fmt, const uint16_t* w, long long nblocks, uint8_t* codes,
                              uint8_t* scales, hipStream_t st);
hipError_t launch_mx_dequantize(int fmt, const uint8_t* codes, const uint8_t* scales,
                                long long nblocks, uint16_t* w, hipStream_t st);
hipError_t launch_combine(const Shape& s, const uint16_t* y, const int32_t* token_row,
                          const float* w, const int32_t* ntok, uint16_t* out, hipStream_t st);
// router top-k: ids [T,K], weights [T,K] from logits fp32 [T,E]
hipError_t launch_router(const Shape& s, const float* logits, const int32_t* ntok, int32_t* ids,
                         float* wts, hipStream_t st);

}  // namespace moe

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
#if defined(__HIPCC__)
typedef __bf16 moe_bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef uint32_t moe_u32x4 __attribute__((ext_vector_type(4)));
typedef float moe_f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float moe_f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

__device__ __forceinline__ float moe_bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.  gfx950's
// v_cvt_pk_bf16_f32 rounds this way (checked bit for bit on the device against
// the integer form u + 0x7fff + ((u >> 16) & 1) over rounding ties,
// subnormals, overflow and NaN).
__device__ __forceinline__ uint16_t moe_f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// two values at once, lo in bits 0-15 (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t moe_f32x2_to_bf16x2(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ int moe_valid_tokens(const int32_t* ntok, int T) {
    if (!ntok) return T;
    int v = *ntok;
    return v < 0 ? 0 : (v > T ? T : v);
}

// In-place exclusive scan of s[0..n) in LDS (one value per slot, any n);
// s[n] receives the total.  s_wave needs blockDim.x/64 ints.  Every thread of
// the block must call it; it ends with a barrier.
__device__ __forceinline__ void moe_block_exclusive_scan(int* s, int n, int* s_wave) {
    const int tid = threadIdx.x, nt = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int per = (n + nt - 1) / nt;
    const int b = tid * per;
    const int e = (b + per < n) ? b + per : n;
    int sum = 0;
    for (int i = b; i < e; ++i) sum += s[i];
    int incl = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int w = 0; w < wave; ++w) run += s_wave[w];
    for (int i = b; i < e; ++i) {
        int v = s[i];
        s[i] = run;
        run += v;
    }
    if (tid == nt - 1) s[n] = run;
    __syncthreads();
}

// Bits needed to tell the expert ids 0..E-1 apart.
__device__ __forceinline__ int moe_expert_bits(int E) { return E <= 1 ? 0 : 32 - __clz(E - 1); }

// The lanes of this wave that hold the same expert id as this lane, as a
// 64-bit lane mask (meaningful for e >= 0; lanes with e < 0 are in no mask).
// One ballot per bit of the id: a valid lane matches when it agrees on every
// one of the nbits low bits, and ids are below 1 << nbits.  The cost is fixed
// however many distinct experts the wave holds.
__device__ __forceinline__ unsigned long long moe_match_mask(int e, int nbits) {
    unsigned long long m = __ballot(e >= 0);
    for (int b = 0; b < nbits; ++b) {
        const int bit = (e >> b) & 1;
        const unsigned long long v = __ballot(bit);
        m &= bit ? v : ~v;
    }
    return m;
}

#endif
