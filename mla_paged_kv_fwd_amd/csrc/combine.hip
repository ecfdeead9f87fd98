// Split-KV combine: merges the partial results of a request's split slots by
// their log-sum-exp.  For slots s with normalised outputs o_s and lse_s:
//   lse = m + ln sum_s exp(lse_s - m),  m = max_s lse_s
//   out = sum_s exp(lse_s - lse) * o_s
// Slots with lse_s = -inf carry no keys and get weight 0.
#include <math.h>

#include "common.h"

namespace mla {

namespace {

constexpr int kCombineThreads = 256;
constexpr int kRowsPerBlock = 4;  // 64 threads x 8 dims per row

__device__ __forceinline__ unsigned short bf16_bits(float f) {
    return __builtin_bit_cast(unsigned short, (__bf16)f);
}

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const int32_t *__restrict__ split_base, int M, const float *__restrict__ o_part,
    const float *__restrict__ lse_part, uint16_t *__restrict__ out, float *__restrict__ lse) {
    const int b = blockIdx.x;
    const int base = split_base[b];
    const int ns = split_base[b + 1] - base;
    if (ns == 1) return;  // written directly by the attention kernel
    const int r = blockIdx.y * kRowsPerBlock + (threadIdx.x >> 6);
    if (r >= M) return;
    const int d = (threadIdx.x & 63) * 8;
    uint16_t *dst = out + ((int64_t)b * M + r) * kDV + d;

    float mx = -INFINITY;
    for (int s = 0; s < ns; ++s) mx = fmaxf(mx, lse_part[(int64_t)(base + s) * M + r]);
    if (mx == -INFINITY) {  // no pages, or no visible key in any slot
        *(u32x4 *)dst = (u32x4){0u, 0u, 0u, 0u};
        if (d == 0) lse[(int64_t)b * M + r] = -INFINITY;
        return;
    }
    float z = 0.f;
    for (int s = 0; s < ns; ++s) z += expf(lse_part[(int64_t)(base + s) * M + r] - mx);
    const float lse_all = mx + logf(z);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < ns; ++s) {
        const float ls = lse_part[(int64_t)(base + s) * M + r];
        if (ls == -INFINITY) continue;
        const float wgt = expf(ls - lse_all);
        const float *src = o_part + ((int64_t)(base + s) * M + r) * kDV + d;
        const f32x4 v0 = *(const f32x4 *)src;
        const f32x4 v1 = *(const f32x4 *)(src + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[e] += wgt * v0[e];
            acc[4 + e] += wgt * v1[e];
        }
    }
    unsigned pk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        pk[e] = (unsigned)bf16_bits(acc[2 * e]) | ((unsigned)bf16_bits(acc[2 * e + 1]) << 16);
    *(u32x4 *)dst = (u32x4){pk[0], pk[1], pk[2], pk[3]};
    if (d == 0) lse[(int64_t)b * M + r] = lse_all;
}

}  // namespace

hipError_t launch_combine(const int32_t *split_base, int batch, int M, const float *o_part,
                          const float *lse_part, uint16_t *out, float *lse, hipStream_t stream) {
    const dim3 grid(batch, (M + kRowsPerBlock - 1) / kRowsPerBlock), block(kCombineThreads);
    hipLaunchKernelGGL(combine_kernel, grid, block, 0, stream, split_base, M, o_part, lse_part,
                       out, lse);
    return hipGetLastError();
}

}  // namespace mla
