// Sparse decode, first stage: each query token (b, i) attends only to the
// cached tokens its list names (DeepSeek KB page, "Key Contributions": the
// FP8 cache serves a sparse decode kernel; the list comes from an indexer the
// pages do not describe).  The list of (b, i) is indices[b][i][0 .. n) with n
// the position of its first negative entry (or topk).
//
// Two kernels turn the lists into an ordinary paged decode problem over
// batch * s_q pseudo-requests of one query token each:
//   - sparse_prep_kernel: per pseudo-request, its list length n (the first
//     negative entry) and a block table onto the gathered pages;
//   - sparse_gather_kernel: one wave per list entry copies the named token's
//     row (bf16, 1152 B) or record (FP8, 656 B) from the paged cache into the
//     gathered cache, entry p of pseudo-request r at slot p of its pages.
// The planner, the decode kernels and the combine then run unchanged.
#include "common.h"

namespace mla {

namespace {

constexpr int kPrepThreads = 256;
constexpr int kGatherRowsPerBlock = 4;

__global__ __launch_bounds__(kPrepThreads) void sparse_prep_kernel(
    const int32_t *__restrict__ indices, int topk, int pages_per, int32_t *__restrict__ lens,
    int32_t *__restrict__ gathered_bt) {
    __shared__ int first_neg[kPrepThreads / 64];
    const int r = blockIdx.x, tid = threadIdx.x;
    const int32_t *list = indices + (int64_t)r * topk;
    int n = topk;
    for (int p = tid; p < topk; p += kPrepThreads)
        if (list[p] < 0) {
            n = p;
            break;
        }
    // minimum over the work-group
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) n = min(n, __shfl_xor(n, m));
    if ((tid & 63) == 0) first_neg[tid >> 6] = n;
    __syncthreads();
    if (tid == 0) {
        int v = first_neg[0];
        for (int k = 1; k < kPrepThreads / 64; ++k) v = min(v, first_neg[k]);
        lens[r] = v;
    }
    for (int j = tid; j < pages_per; j += kPrepThreads)
        gathered_bt[(int64_t)r * pages_per + j] = r * pages_per + j;
}

template <bool FP8>
__global__ __launch_bounds__(64 * kGatherRowsPerBlock) void sparse_gather_kernel(
    const unsigned char *__restrict__ kv, const int32_t *__restrict__ block_table,
    int64_t bt_stride, const int32_t *__restrict__ indices, int s_q, int topk, int pages_per,
    unsigned char *__restrict__ gathered) {
    constexpr int kBytes = FP8 ? kTokBytesFp8 : kTokBytesBf16;
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.y;  // pseudo-request b * s_q + i
    const int p = blockIdx.x * kGatherRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (p >= topk) return;
    const int idx = indices[(int64_t)r * topk + p];
    if (idx < 0) return;  // past the list's end: never read by the decode
    const int b = r / s_q;
    const int64_t phys = block_table[(int64_t)b * bt_stride + idx / kPage];
    const u32x4 *src = (const u32x4 *)(kv + (phys * kPage + idx % kPage) * kBytes);
    u32x4 *dst = (u32x4 *)(gathered + ((int64_t)r * pages_per * kPage + p) * kBytes);
    for (int c = lane; c < kBytes / 16; c += 64) dst[c] = src[c];
}

}  // namespace

hipError_t launch_sparse_prep(const int32_t *indices, int rows, int topk, int pages_per,
                              int32_t *lens, int32_t *gathered_bt, hipStream_t stream) {
    hipLaunchKernelGGL(sparse_prep_kernel, dim3(rows), dim3(kPrepThreads), 0, stream, indices, topk,
                       pages_per, lens, gathered_bt);
    return hipGetLastError();
}

hipError_t launch_sparse_gather(const unsigned char *kv, bool fp8, const int32_t *block_table,
                                int64_t bt_stride, const int32_t *indices, int batch, int s_q,
                                int topk, int pages_per, unsigned char *gathered,
                                hipStream_t stream) {
    const dim3 grid((unsigned)((topk + kGatherRowsPerBlock - 1) / kGatherRowsPerBlock),
                    (unsigned)(batch * s_q));
    const dim3 block(64 * kGatherRowsPerBlock);
    if (fp8)
        hipLaunchKernelGGL(sparse_gather_kernel<true>, grid, block, 0, stream, kv, block_table,
                           bt_stride, indices, s_q, topk, pages_per, gathered);
    else
        hipLaunchKernelGGL(sparse_gather_kernel<false>, grid, block, 0, stream, kv, block_table,
                           bt_stride, indices, s_q, topk, pages_per, gathered);
    return hipGetLastError();
}

}  // namespace mla
