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

    // Slots are merged four at a time: a chunk's lse values and partial
    // outputs are loaded together, then merged into a running (max, sum,
    // output) with a rescale when the max grows, so each chunk costs one
    // memory round trip.  A slot with lse = -inf gets weight 0 whatever it
    // holds.
    const float *lrow = lse_part + (int64_t)base * M + r;
    const float *orow = o_part + ((int64_t)base * M + r) * kDV + d;
    const int64_t ostride = (int64_t)M * kDV;
    float mx = -INFINITY, z = 0.f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < ns; s0 += 4) {
        float ls[4];
        f32x4 v0[4], v1[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int s = s0 + k < ns ? s0 + k : ns - 1;
            ls[k] = s0 + k < ns ? lrow[(int64_t)s * M] : -INFINITY;
            v0[k] = *(const f32x4 *)(orow + s * ostride);
            v1[k] = *(const f32x4 *)(orow + s * ostride + 4);
        }
        const float mc = fmaxf(fmaxf(ls[0], ls[1]), fmaxf(ls[2], ls[3]));
        if (mc == -INFINITY) continue;  // no keys in this chunk
        const float mn = fmaxf(mx, mc);
        const float sc = expf(mx - mn);  // 0 while nothing has been merged
        z *= sc;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] *= sc;
        mx = mn;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float e = expf(ls[k] - mx);  // 0 for an empty slot
            z += e;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[j] += ls[k] == -INFINITY ? 0.f : e * v0[k][j];
                acc[4 + j] += ls[k] == -INFINITY ? 0.f : e * v1[k][j];
            }
        }
    }
    if (mx == -INFINITY) {  // no pages, or no visible key in any slot
        *(u32x4 *)dst = (u32x4){0u, 0u, 0u, 0u};
        if (d == 0) lse[(int64_t)b * M + r] = -INFINITY;
        return;
    }
    const float lse_all = mx + logf(z);
    const float inv_z = 1.f / z;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= inv_z;
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
