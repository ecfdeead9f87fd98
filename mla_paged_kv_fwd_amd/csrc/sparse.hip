// Sparse decode, first stage: each query token (b, i) attends only to the
// cached tokens its list names (DeepSeek KB page, "Key Contributions": the
// FP8 cache serves a sparse decode kernel; the list comes from an indexer the
// pages do not describe).  The list of (b, i) is indices[b][i][0 .. n) with n
// the position of its first negative entry (or topk).
//
// Each query token becomes a pseudo-request of one query token whose keys
// are its listed tokens, batch * s_q of them, planned and merged like any
// decode.  sparse_ids_kernel writes, per pseudo-request, its list length n
// (the position of the first negative entry) and the cache token id
// (page * 64 + slot) of each listed position; the 64-row kernels, in their
// token-list mode, then read every listed row or record straight from its
// page.  List entries at or past the first negative one are never
// dereferenced.
#include "common.h"

namespace mla {

namespace {

constexpr int kPrepThreads = 256;

constexpr int kPerThread = 8;  // list entries each thread loads before using any

constexpr int kChunk = kPrepThreads * kPerThread;

// Length of list r: the position of its first negative entry, else topk.
// All kPrepThreads threads; the result in every thread.  Every thread loads
// its kPerThread entries of a chunk at once (no early exit), so a chunk of
// kChunk entries costs one memory round trip.  The first chunk's entries are
// returned in first[] (entry k * kPrepThreads + tid in first[k]), so that a
// list of at most kChunk entries is read once.
__device__ __forceinline__ int list_length(const int32_t *list, int topk, int *scratch,
                                           int (&first)[kPerThread]) {
    const int tid = threadIdx.x;
    int n = topk;
    for (int p0 = 0; p0 < topk; p0 += kChunk) {
        int v[kPerThread];
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
            const int p = p0 + k * kPrepThreads + tid;
            v[k] = p < topk ? list[p] : 0;
        }
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
            const int p = p0 + k * kPrepThreads + tid;
            if (v[k] < 0) n = min(n, p);
            if (p0 == 0) first[k] = v[k];
        }
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
// Per chunk, the list entries are loaded (the first chunk's are already in
// registers), then their block-table entries, then the ids are stored.
__global__ __launch_bounds__(kPrepThreads) void sparse_ids_kernel(
    const int32_t *__restrict__ indices, const int32_t *__restrict__ block_table,
    int64_t bt_stride, int s_q, int topk, int tok_per, int32_t *__restrict__ lens,
    int32_t *__restrict__ ids) {
    __shared__ int scratch[kPrepThreads / 64];
    const int r = blockIdx.x, tid = threadIdx.x;
    const int32_t *list = indices + (int64_t)r * topk;
    int first[kPerThread];
    const int n = list_length(list, topk, scratch, first);
    if (tid == 0) lens[r] = n;
    const int32_t *bt = block_table + (int64_t)(r / s_q) * bt_stride;
    int32_t *dst = ids + (int64_t)r * tok_per;
    for (int p0 = 0; p0 < tok_per; p0 += kChunk) {
        int pos[kPerThread], page[kPerThread];
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
            const int p = p0 + k * kPrepThreads + tid;
            pos[k] = p < n ? (p0 == 0 ? first[k] : list[p]) : -1;
        }
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) page[k] = pos[k] >= 0 ? bt[pos[k] / kPage] : 0;
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
            const int p = p0 + k * kPrepThreads + tid;
            if (p < tok_per) dst[p] = pos[k] >= 0 ? page[k] * kPage + pos[k] % kPage : 0;
        }
    }
}

}  // namespace

hipError_t launch_sparse_ids(const int32_t *indices, const int32_t *block_table,
                             int64_t bt_stride, int rows, int s_q, int topk, int tok_per,
                             int32_t *lens, int32_t *ids, hipStream_t stream) {
    hipLaunchKernelGGL(sparse_ids_kernel, dim3(rows), dim3(kPrepThreads), 0, stream, indices,
                       block_table, bt_stride, s_q, topk, tok_per, lens, ids);
    return hipGetLastError();
}

}  // namespace mla
