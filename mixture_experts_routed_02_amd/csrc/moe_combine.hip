// Weighted top-k combine back to token order (TileOps PR #1738 "[Refactor]
// [MoE] Separate dispatched expert compute", Summary: the routing weights are
// applied outside expert compute; FlashInfer PR #3980, commit notes on the
// kernel API migration, launch/output: a single (tokens, hidden) output with
// the top-k reduction done inside the layer).
//
// out[t,:] = bf16( sum over j = 0..K-1 with token_row[t*K+j] >= 0 of
//                  w[t,j] * y[token_row[t*K+j], :] ),  fp32 fused multiply-adds
// in increasing j, one round-to-nearest-even at the end; a zero row when no
// assignment of t is valid; rows t >= T_v are not written.  Each token is
// owned by one workgroup, so there are no atomics and the result is
// bit-reproducible.  Loads and stores are 16 bytes (8 bf16) per lane.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kCombineThreads = 256;
constexpr int kMaxTopK = 64;

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const uint4* __restrict__ y, const int32_t* __restrict__ token_row,
    const float* __restrict__ w, const int32_t* __restrict__ ntok, int T, int K, int vec,
    uint4* __restrict__ out) {
    __shared__ int s_row[kMaxTopK];
    __shared__ float s_w[kMaxTopK];
    const int tv = moe_valid_tokens(ntok, T);
    for (int t = blockIdx.x; t < tv; t += gridDim.x) {
        if (threadIdx.x < K) {
            s_row[threadIdx.x] = token_row[(long long)t * K + threadIdx.x];
            s_w[threadIdx.x] = w[(long long)t * K + threadIdx.x];
        }
        __syncthreads();
        for (int c = threadIdx.x; c < vec; c += blockDim.x) {
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int j = 0; j < K; ++j) {
                const int r = s_row[j];
                if (r < 0) continue;
                const float wj = s_w[j];
                const uint4 v = y[(long long)r * vec + c];
                const uint32_t pk[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[2 * q] = fmaf(wj, __uint_as_float(pk[q] << 16), acc[2 * q]);
                    acc[2 * q + 1] = fmaf(wj, __uint_as_float(pk[q] & 0xffff0000u), acc[2 * q + 1]);
                }
            }
            uint4 o;
            o.x = (uint32_t)moe_f32_to_bf16(acc[0]) | ((uint32_t)moe_f32_to_bf16(acc[1]) << 16);
            o.y = (uint32_t)moe_f32_to_bf16(acc[2]) | ((uint32_t)moe_f32_to_bf16(acc[3]) << 16);
            o.z = (uint32_t)moe_f32_to_bf16(acc[4]) | ((uint32_t)moe_f32_to_bf16(acc[5]) << 16);
            o.w = (uint32_t)moe_f32_to_bf16(acc[6]) | ((uint32_t)moe_f32_to_bf16(acc[7]) << 16);
            out[(long long)t * vec + c] = o;
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_combine(const Shape& s, const uint16_t* y, const int32_t* token_row,
                          const float* w, const int32_t* ntok, uint16_t* out, hipStream_t st) {
    int grid = s.T < 8 * kNumCUs ? s.T : 8 * kNumCUs;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(combine_kernel, dim3(grid), dim3(kCombineThreads), 0, st,
                       reinterpret_cast<const uint4*>(y), token_row, w, ntok, s.T, s.K, s.H / 8,
                       reinterpret_cast<uint4*>(out));
    return hipGetLastError();
}

}  // namespace moe
