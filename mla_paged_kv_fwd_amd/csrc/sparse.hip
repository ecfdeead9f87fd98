// Sparse decode, first stage: each query token (b, i) attends only to the
// cached tokens its list names (DeepSeek KB page, "Key Contributions": the
// FP8 cache serves a sparse decode kernel; the list comes from an indexer the
// pages do not describe).  The list of (b, i) is indices[b][i][0 .. n) with n
// the position of its first negative entry (or topk).
//
// Each query token becomes a pseudo-request of one query token whose keys
// are its listed tokens, batch * s_q of them, planned and merged like any
// decode.  Two ways to feed them to the decode kernels:
//   - token ids (64-row kernels, h_q >= 32): sparse_ids_kernel writes, per
//     pseudo-request, its list length n and the cache token id
//     (page * 64 + slot) of each listed position; the kernels read every
//     listed row or record straight from its page;
//   - gathered copy (16-row kernel, h_q = 16): sparse_prep_kernel writes n
//     and a block table onto gathered pages, and sparse_gather_kernel copies
//     each listed row (bf16, 1152 B) or record (FP8, 656 B) there, one wave
//     per entry; the kernels then decode the copy as an ordinary paged cache.
// List entries at or past the first negative one are never dereferenced.
#include "common.h"

namespace mla {

namespace {

constexpr int kPrepThreads = 256;
constexpr int kGatherRowsPerBlock = 4;

// Length of list r: the position of its first negative entry, else topk.
// All kPrepThreads threads; the result in every thread.
__device__ __forceinline__ int list_length(const int32_t *list, int topk, int *scratch) {
    const int tid = threadIdx.x;
    int n = topk;
    for (int p = tid; p < topk; p += kPrepThreads)
        if (list[p] < 0) {
            n = p;
            break;
        }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) n = min(n, __shfl_xor(n, m));
    if ((tid & 63) == 0) scratch[tid >> 6] = n;
    __syncthreads();
    int v = scratch[0];
#pragma unroll
    for (int k = 1; k < kPrepThreads / 64; ++k) v = min(v, scratch[k]);
    return v;
}

// One work-group per pseudo-request r = b * s_q + i: lens[r] = n and
// ids[r][p] = the cache token id of entry p for p < n, 0 for n <= p < tok_per.
__global__ __launch_bounds__(kPrepThreads) void sparse_ids_kernel(
    const int32_t *__restrict__ indices, const int32_t *__restrict__ block_table,
    int64_t bt_stride, int s_q, int topk, int tok_per, int32_t *__restrict__ lens,
    int32_t *__restrict__ ids) {
    __shared__ int scratch[kPrepThreads / 64];
    const int r = blockIdx.x, tid = threadIdx.x;
    const int32_t *list = indices + (int64_t)r * topk;
    const int n = list_length(list, topk, scratch);
    if (tid == 0) lens[r] = n;
    const int32_t *bt = block_table + (int64_t)(r / s_q) * bt_stride;
    int32_t *dst = ids + (int64_t)r * tok_per;
    for (int p = tid; p < tok_per; p += kPrepThreads) {
        int id = 0;
        if (p < n) {
            const int pos = list[p];
            id = bt[pos / kPage] * kPage + pos % kPage;
        }
        dst[p] = id;
    }
}

__global__ __launch_bounds__(kPrepThreads) void sparse_prep_kernel(
    const int32_t *__restrict__ indices, int topk, int pages_per, int32_t *__restrict__ lens,
    int32_t *__restrict__ gathered_bt) {
    __shared__ int scratch[kPrepThreads / 64];
    const int r = blockIdx.x, tid = threadIdx.x;
    const int n = list_length(indices + (int64_t)r * topk, topk, scratch);
    if (tid == 0) lens[r] = n;
    for (int j = tid; j < pages_per; j += kPrepThreads)
        gathered_bt[(int64_t)r * pages_per + j] = r * pages_per + j;
}

template <bool FP8>
__global__ __launch_bounds__(64 * kGatherRowsPerBlock) void sparse_gather_kernel(
    const unsigned char *__restrict__ kv, const int32_t *__restrict__ block_table,
    int64_t bt_stride, const int32_t *__restrict__ indices, const int32_t *__restrict__ lens,
    int s_q, int topk, int pages_per, unsigned char *__restrict__ gathered) {
    constexpr int kBytes = FP8 ? kTokBytesFp8 : kTokBytesBf16;
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.y;  // pseudo-request b * s_q + i
    const int p = blockIdx.x * kGatherRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (p >= lens[r]) return;  // past the list's end: never read by the decode
    const int idx = indices[(int64_t)r * topk + p];
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

hipError_t launch_sparse_ids(const int32_t *indices, const int32_t *block_table,
                             int64_t bt_stride, int rows, int s_q, int topk, int tok_per,
                             int32_t *lens, int32_t *ids, hipStream_t stream) {
    hipLaunchKernelGGL(sparse_ids_kernel, dim3(rows), dim3(kPrepThreads), 0, stream, indices,
                       block_table, bt_stride, s_q, topk, tok_per, lens, ids);
    return hipGetLastError();
}

hipError_t launch_sparse_gather(const unsigned char *kv, bool fp8, const int32_t *block_table,
                                int64_t bt_stride, const int32_t *indices, const int32_t *lens,
                                int batch, int s_q, int topk, int pages_per,
                                unsigned char *gathered, hipStream_t stream) {
    const dim3 grid((unsigned)((topk + kGatherRowsPerBlock - 1) / kGatherRowsPerBlock),
                    (unsigned)(batch * s_q));
    const dim3 block(64 * kGatherRowsPerBlock);
    if (fp8)
        hipLaunchKernelGGL(sparse_gather_kernel<true>, grid, block, 0, stream, kv, block_table,
                           bt_stride, indices, lens, s_q, topk, pages_per, gathered);
    else
        hipLaunchKernelGGL(sparse_gather_kernel<false>, grid, block, 0, stream, kv, block_table,
                           bt_stride, indices, lens, s_q, topk, pages_per, gathered);
    return hipGetLastError();
}

}  // namespace mla
