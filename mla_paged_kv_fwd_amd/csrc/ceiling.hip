// Measured ceilings of the part (gfx950): a plain HBM streaming read and
// back-to-back bf16 MFMA loops.  The decode kernels' roofline fractions are
// quoted against the published peaks and, beside them, against these
// measured rates, which include the clock the part actually holds under
// sustained load.  Not part of the decode path; bench.py loads this library
// on its own.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla_ceiling.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;

// Every thread reads 16-byte vectors at a grid-wide stride, four loads in
// flight, and folds them into one word so that no load is dead.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4 *__restrict__ src,
                                                               int64_t n, unsigned *__restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + 3 * stride < n; i += 4 * stride) {
        const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n; i += stride) acc ^= src[i];
    sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

__device__ __forceinline__ bf16x8 operand(int seed) {
    bf16x8 v;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const unsigned h = (unsigned)(seed * 8 + k) * 2654435761u;
        v[k] = (__bf16)((float)(h >> 20) * (1.0f / 4096.0f) - 0.5f);
    }
    return v;
}

// Four independent accumulator chains per wave, `iters` rounds of one MFMA
// per chain, written as one asm block per round so that the accumulators stay
// in place (each chain's previous MFMA is three MFMAs back, so no result is
// waited for): the matrix unit of each SIMD runs back to back.
template <int kShape>
__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(int iters, float *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const bf16x8 a = operand(lane), b = operand(lane + 64);
    float total = 0.f;
    if constexpr (kShape == 0) {
        f32x4 c0 = {}, c1 = {}, c2 = {}, c3 = {};
        for (int it = 0; it < iters; ++it)
            asm volatile(
                "v_mfma_f32_16x16x32_bf16 %0, %4, %5, %0\n\t"
                "v_mfma_f32_16x16x32_bf16 %1, %4, %5, %1\n\t"
                "v_mfma_f32_16x16x32_bf16 %2, %4, %5, %2\n\t"
                "v_mfma_f32_16x16x32_bf16 %3, %4, %5, %3"
                : "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3)
                : "v"(a), "v"(b));
        asm volatile("s_nop 7\n\ts_nop 7" ::);
        total = c0[0] + c1[1] + c2[2] + c3[3];
    } else {
        f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
        for (int it = 0; it < iters; ++it)
            asm volatile(
                "v_mfma_f32_32x32x16_bf16 %0, %4, %5, %0\n\t"
                "v_mfma_f32_32x32x16_bf16 %1, %4, %5, %1\n\t"
                "v_mfma_f32_32x32x16_bf16 %2, %4, %5, %2\n\t"
                "v_mfma_f32_32x32x16_bf16 %3, %4, %5, %3"
                : "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3)
                : "v"(a), "v"(b));
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::);
        total = c0[0] + c1[5] + c2[10] + c3[15];
    }
    sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = total;
}

int g_cus[64];

int cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
    if (g_cus[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return -1;
        g_cus[dev] = n;
    }
    return g_cus[dev];
}

}  // namespace

extern "C" {

int mla_ceiling_blocks(int blocks_per_cu) {
    const int cus = cu_count();
    if (cus <= 0 || blocks_per_cu < 1 || blocks_per_cu > 64) return -1;
    return cus * blocks_per_cu;
}

int mla_ceiling_stream_read(const void *buf, size_t bytes, int blocks_per_cu, unsigned *sink,
                            void *stream) {
    const int grid = mla_ceiling_blocks(blocks_per_cu);
    if (!buf || !sink || grid <= 0 || bytes < 16 || (bytes & 15) != 0 || ((uintptr_t)buf & 15) != 0)
        return -1;
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                       (const u32x4 *)buf, (int64_t)(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int mla_ceiling_mfma(int shape, int iters, int blocks_per_cu, float *sink, void *stream) {
    const int grid = mla_ceiling_blocks(blocks_per_cu);
    if (!sink || grid <= 0 || iters < 1 || (shape != 0 && shape != 1)) return -1;
    if (shape == 0)
        hipLaunchKernelGGL(mfma_loop_kernel<0>, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                           iters, sink);
    else
        hipLaunchKernelGGL(mfma_loop_kernel<1>, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                           iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

double mla_ceiling_mfma_flops(int shape, int iters, int blocks_per_cu) {
    const int grid = mla_ceiling_blocks(blocks_per_cu);
    if (grid <= 0 || iters < 1 || (shape != 0 && shape != 1)) return -1.0;
    const double per = shape == 0 ? 2.0 * 16 * 16 * 32 : 2.0 * 32 * 32 * 16;
    return (double)grid * (kThreads / 64) * 4.0 * iters * per;
}

}  // extern "C"
