// Device-side checks of the caller's device data, which the decode kernels
// take on trust: block-table entries against the page pool, request lengths
// against the table's width, and sparse list entries against the table.  A
// check reads only table entries inside the table, so it is safe on the very
// inputs it rejects.
//
// result (device, 2 x uint64, written by the call): result[0] = number of bad
// requests (bad lists for the sparse check); result[1] = the smallest key
// (request << 32) | where over the bad ones, where = the first bad logical
// page (block-table check), the first bad list position (sparse check), or
// 0xFFFFFFFF for a bad length; ~0 if nothing is bad.
#include <stdint.h>

#include "common.h"

namespace mla {

namespace {

constexpr int kCheckThreads = 256;
constexpr unsigned kBadLength = 0xFFFFFFFFu;

__global__ void check_init_kernel(unsigned long long *result) {
    if (threadIdx.x == 0) {
        result[0] = 0ull;
        result[1] = ~0ull;
    }
}

// Work-group minimum of v; the result in every thread.
__device__ __forceinline__ int block_min(int v, int *scratch) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v = min(v, __shfl_xor(v, m));
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
    __syncthreads();
    int r = scratch[0];
#pragma unroll
    for (int k = 1; k < kCheckThreads / 64; ++k) r = min(r, scratch[k]);
    return r;
}

__device__ __forceinline__ void report(unsigned long long *result, int r, unsigned where) {
    atomicAdd(&result[0], 1ull);
    atomicMin(&result[1], ((unsigned long long)r << 32) | where);
}

// One work-group per request.
__global__ __launch_bounds__(kCheckThreads) void check_block_table_kernel(
    const int32_t *__restrict__ seqlens, const int32_t *__restrict__ block_table,
    int64_t bt_stride, int64_t num_pages, unsigned long long *result) {
    __shared__ int scratch[kCheckThreads / 64];
    const int b = blockIdx.x;
    const int64_t L = seqlens[b];
    const int64_t n = (L + kPage - 1) / kPage;
    if (L < 0 || n > bt_stride) {
        if (threadIdx.x == 0) report(result, b, kBadLength);
        return;
    }
    const int32_t *bt = block_table + (int64_t)b * bt_stride;
    int first = 0x7FFFFFFF;
    for (int j = threadIdx.x; j < n; j += kCheckThreads) {
        const int p = bt[j];
        if ((p < 0 || p >= num_pages) && j < first) first = j;
    }
    first = block_min(first, scratch);
    if (threadIdx.x == 0 && first != 0x7FFFFFFF) report(result, b, (unsigned)first);
}

// One work-group per list r = b * s_q + i: entries before the first negative
// one must name a logical page inside the table whose entry is a pool page.
__global__ __launch_bounds__(kCheckThreads) void check_sparse_kernel(
    const int32_t *__restrict__ block_table, int64_t bt_stride, int64_t num_pages,
    const int32_t *__restrict__ indices, int s_q, int topk, unsigned long long *result) {
    __shared__ int scratch[kCheckThreads / 64];
    const int r = blockIdx.x;
    const int32_t *list = indices + (int64_t)r * topk;
    int n = topk;
    for (int p = threadIdx.x; p < topk; p += kCheckThreads)
        if (list[p] < 0) {
            n = p;
            break;
        }
    n = block_min(n, scratch);
    __syncthreads();  // scratch is reused
    const int32_t *bt = block_table + (int64_t)(r / s_q) * bt_stride;
    int first = 0x7FFFFFFF;
    for (int p = threadIdx.x; p < n; p += kCheckThreads) {
        const int j = list[p] / kPage;
        bool bad = j >= bt_stride;
        if (!bad) {
            const int page = bt[j];
            bad = page < 0 || page >= num_pages;
        }
        if (bad && p < first) first = p;
    }
    first = block_min(first, scratch);
    if (threadIdx.x == 0 && first != 0x7FFFFFFF) report(result, r, (unsigned)first);
}

}  // namespace

hipError_t launch_check_block_table(const int32_t *seqlens, int batch, const int32_t *block_table,
                                    int64_t bt_stride, int64_t num_pages,
                                    unsigned long long *result, hipStream_t stream) {
    hipLaunchKernelGGL(check_init_kernel, dim3(1), dim3(64), 0, stream, result);
    hipLaunchKernelGGL(check_block_table_kernel, dim3(batch), dim3(kCheckThreads), 0, stream,
                       seqlens, block_table, bt_stride, num_pages, result);
    return hipGetLastError();
}

hipError_t launch_check_sparse(const int32_t *block_table, int64_t bt_stride, int64_t num_pages,
                               const int32_t *indices, int rows, int s_q, int topk,
                               unsigned long long *result, hipStream_t stream) {
    hipLaunchKernelGGL(check_init_kernel, dim3(1), dim3(64), 0, stream, result);
    hipLaunchKernelGGL(check_sparse_kernel, dim3(rows), dim3(kCheckThreads), 0, stream,
                       block_table, bt_stride, num_pages, indices, s_q, topk, result);
    return hipGetLastError();
}

}  // namespace mla
