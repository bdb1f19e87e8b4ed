// Router top-k, the step ahead of dispatch (TileOps PR #1738, Summary: the
// routing weights are produced outside expert compute and travel beside the
// ids).  For every valid token t (t < T_v) and its E router logits:
//   ids[t, 0..K-1]  the K largest logits in decreasing order, equal values in
//                   increasing expert index;
//   w[t, j]         exp(l_j - l_0) / sum_{i<K} exp(l_i - l_0), l_j the j-th
//                   selected logit (a softmax over the selected K), fp32, the
//                   sum taken in increasing j;
// rows t >= T_v are not written.
//
// One wave per token.  Lane l holds logits l, l+64, ... as 64-bit keys whose
// high word orders the fp32 value (sign-magnitude flipped to an unsigned
// order, -0 folded onto +0) and whose low word is ~index, so the largest key
// is the largest value with, among equal values, the lowest index.  Each of
// the K rounds takes the wave maximum with xor shuffles and clears the
// winner; lane j keeps round j's pick.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouterWaves = 4;

__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t b = __float_as_uint(v);
    if (b == 0x80000000u) b = 0u;   // -0 == +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_value(unsigned long long k) {
    const uint32_t o = (uint32_t)(k >> 32);
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// PER = logits per lane, E <= 64 * PER
template <int PER>
__global__ __launch_bounds__(64 * kRouterWaves) void router_topk_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ ntok, int T, int E, int K,
    int32_t* __restrict__ ids, float* __restrict__ wts) {
    const int lane = threadIdx.x & 63;
    const int tv = moe_valid_tokens(ntok, T);
    for (int t = blockIdx.x * kRouterWaves + (threadIdx.x >> 6); t < tv;
         t += gridDim.x * kRouterWaves) {
        const float* row = logits + (size_t)t * E;
        unsigned long long key[PER];   // 0 = empty (no real key is 0: ~index is never 0)
#pragma unroll
        for (int c = 0; c < PER; ++c) {
            const int e = c * 64 + lane;
            key[c] = e < E ? (((unsigned long long)order_key(row[e]) << 32) | (uint32_t)~(uint32_t)e)
                           : 0ull;
        }
        int my_e = 0;
        float my_v = 0.f, v0 = 0.f;
        for (int j = 0; j < K; ++j) {
            unsigned long long best = key[0];
#pragma unroll
            for (int c = 1; c < PER; ++c) best = key[c] > best ? key[c] : best;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const unsigned long long other = __shfl_xor(best, o, 64);
                best = other > best ? other : best;
            }
            const int e = (int)~(uint32_t)best;
#pragma unroll
            for (int c = 0; c < PER; ++c)
                if (c * 64 + lane == e) key[c] = 0ull;
            const float v = key_value(best);
            if (j == 0) v0 = v;
            if (lane == j) {
                my_e = e;
                my_v = v;
            }
        }
        const float ex = lane < K ? expf(my_v - v0) : 0.f;
        float sum = 0.f;
        for (int j = 0; j < K; ++j) sum += __shfl(ex, j, 64);   // increasing j
        if (lane < K) {
            ids[(size_t)t * K + lane] = my_e;
            wts[(size_t)t * K + lane] = ex / sum;
        }
    }
}

}  // namespace

hipError_t launch_router(const Shape& s, const float* logits, const int32_t* ntok, int32_t* ids,
                         float* wts, hipStream_t st) {
    long long blocks = ((long long)s.T + kRouterWaves - 1) / kRouterWaves;
    if (blocks > 8 * kNumCUs) blocks = 8 * kNumCUs;
    if (blocks < 1) blocks = 1;
    const dim3 grid((unsigned)blocks), block(64 * kRouterWaves);
    if (s.E <= 64)
        hipLaunchKernelGGL(router_topk_kernel<1>, grid, block, 0, st, logits, ntok, s.T, s.E, s.K, ids, wts);
    else if (s.E <= 128)
        hipLaunchKernelGGL(router_topk_kernel<2>, grid, block, 0, st, logits, ntok, s.T, s.E, s.K, ids, wts);
    else if (s.E <= 256)
        hipLaunchKernelGGL(router_topk_kernel<4>, grid, block, 0, st, logits, ntok, s.T, s.E, s.K, ids, wts);
    else
        hipLaunchKernelGGL(router_topk_kernel<8>, grid, block, 0, st, logits, ntok, s.T, s.E, s.K, ids, wts);
    return hipGetLastError();
}

}  // namespace moe
