// Split-KV planner: device kernel and its host twin.  Both evaluate the same
// PlanView functions on the same integer prefix sums, so they agree bit for bit.
#include <vector>

#include "common.h"

namespace mla {

namespace {

constexpr int kPlanThreads = 1024;

// Block-wide exclusive scan of one int per thread (kPlanThreads threads).
__device__ int block_exclusive_scan(int v, int *scratch, int *total) {
    const int t = threadIdx.x;
    scratch[t] = v;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
        int add = (t >= off) ? scratch[t - off] : 0;
        __syncthreads();
        scratch[t] += add;
        __syncthreads();
    }
    int incl = scratch[t];
    *total = scratch[kPlanThreads - 1];
    __syncthreads();
    return incl - v;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t *__restrict__ seqlens,
                                                            int batch, int c, int num_parts,
                                                            int32_t *__restrict__ meta,
                                                            int32_t *__restrict__ split_base) {
    __shared__ int32_t pages_pre[kMaxBatch + 1];
    __shared__ int32_t nonempty_pre[kMaxBatch + 1];
    __shared__ int scratch[kPlanThreads];
    const int t = threadIdx.x;
    const int chunk = (batch + kPlanThreads - 1) / kPlanThreads;
    const int b_lo = min(batch, t * chunk), b_hi = min(batch, b_lo + chunk);

    int my_pages = 0, my_nonempty = 0;
    for (int b = b_lo; b < b_hi; ++b) {
        int L = seqlens[b];
        int n = L > 0 ? (L + kPage - 1) / kPage : 0;
        my_pages += n;
        my_nonempty += n > 0;
    }
    int tot_pages, tot_nonempty;
    int pages_off = block_exclusive_scan(my_pages, scratch, &tot_pages);
    int ne_off = block_exclusive_scan(my_nonempty, scratch, &tot_nonempty);
    for (int b = b_lo; b < b_hi; ++b) {
        pages_pre[b] = pages_off;
        nonempty_pre[b] = ne_off;
        int L = seqlens[b];
        int n = L > 0 ? (L + kPage - 1) / kPage : 0;
        pages_off += n;
        ne_off += n > 0;
    }
    if (t == 0) {
        pages_pre[batch] = tot_pages;
        nonempty_pre[batch] = tot_nonempty;
    }
    __syncthreads();

    PlanView v;
    v.pages_pre = pages_pre;
    v.nonempty_pre = nonempty_pre;
    v.batch = batch;
    v.c = c;
    v.total = (int64_t)tot_pages + (int64_t)c * tot_nonempty;
    v.parts_eff = v.total < num_parts ? v.total : num_parts;

    for (int p = t; p < num_parts; p += kPlanThreads) {
        int32_t row[kMetaInts];
        v.part_row(p, row);
        for (int k = 0; k < kMetaInts; ++k) meta[p * kMetaInts + k] = row[k];
    }

    int my_splits = 0;
    for (int b = b_lo; b < b_hi; ++b) my_splits += v.splits_of(b);
    int tot_splits;
    int off = block_exclusive_scan(my_splits, scratch, &tot_splits);
    for (int b = b_lo; b < b_hi; ++b) {
        split_base[b] = off;
        off += v.splits_of(b);
    }
    if (t == 0) split_base[batch] = tot_splits;
}

}  // namespace

hipError_t launch_plan(const int32_t *seqlens, int batch, int c, int num_parts, int32_t *meta,
                       int32_t *split_base, hipStream_t stream) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, seqlens, batch, c,
                       num_parts, meta, split_base);
    return hipGetLastError();
}

void plan_host(const int32_t *seqlens, int batch, int c, int num_parts, int32_t *meta,
               int32_t *split_base) {
    std::vector<int32_t> pages_pre(batch + 1, 0), nonempty_pre(batch + 1, 0);
    for (int b = 0; b < batch; ++b) {
        int L = seqlens[b];
        int n = L > 0 ? (L + kPage - 1) / kPage : 0;
        pages_pre[b + 1] = pages_pre[b] + n;
        nonempty_pre[b + 1] = nonempty_pre[b] + (n > 0);
    }
    PlanView v;
    v.pages_pre = pages_pre.data();
    v.nonempty_pre = nonempty_pre.data();
    v.batch = batch;
    v.c = c;
    v.total = (int64_t)pages_pre[batch] + (int64_t)c * nonempty_pre[batch];
    v.parts_eff = v.total < num_parts ? v.total : num_parts;
    for (int p = 0; p < num_parts; ++p) v.part_row(p, meta + (size_t)p * kMetaInts);
    split_base[0] = 0;
    for (int b = 0; b < batch; ++b) split_base[b + 1] = split_base[b] + v.splits_of(b);
}

}  // namespace mla
