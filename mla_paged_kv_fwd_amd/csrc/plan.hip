// Split-KV planner: device kernel and its host twin.  Both evaluate the same
// PlanView functions on the same integer prefix sums, so they agree bit for bit.
#include <vector>

#include "common.h"

namespace mla {

namespace {

constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / 64;

// Inclusive prefix sum across the 64 lanes of a wave with row shifts and row
// broadcasts (DPP): sums within each 16-lane row, then row 0's total into row
// 1 and row 2's into row 3, then lanes 0..31's total into rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// Block-wide inclusive scan of two ints per thread: a scan within each wave,
// then every thread adds the totals of the waves before it.  Two barriers.
// *total receives the block-wide sums.
__device__ int2 block_inclusive_scan2(int2 v, int2 *wave_tot, int2 *total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    v.x = wave_inclusive_scan(v.x);
    v.y = wave_inclusive_scan(v.y);
    if (lane == 63) wave_tot[wv] = v;
    __syncthreads();
    int2 pre = {0, 0}, tot = {0, 0};
#pragma unroll
    for (int k = 0; k < kPlanWaves; ++k) {
        const int2 w = wave_tot[k];
        if (k < wv) {
            pre.x += w.x;
            pre.y += w.y;
        }
        tot.x += w.x;
        tot.y += w.y;
    }
    __syncthreads();  // wave_tot may be reused
    *total = tot;
    return {v.x + pre.x, v.y + pre.y};
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t *__restrict__ seqlens,
                                                            int batch, int c, int num_parts,
                                                            int32_t *__restrict__ meta,
                                                            int32_t *__restrict__ split_base) {
    __shared__ int32_t pages_pre[kMaxBatch + 1];
    __shared__ int32_t nonempty_pre[kMaxBatch + 1];
    __shared__ int2 wave_tot[kPlanWaves];
    const int t = threadIdx.x;
    // thread t owns requests b_lo .. b_hi - 1; their page counts wait in
    // pages_pre until the scan has produced the offsets
    const int chunk = (batch + kPlanThreads - 1) / kPlanThreads;
    const int b_lo = min(batch, t * chunk), b_hi = min(batch, b_lo + chunk);

    int2 mine = {0, 0};  // (pages, non-empty requests)
    for (int b = b_lo; b < b_hi; ++b) {
        const int L = seqlens[b];
        const int n = L > 0 ? (L + kPage - 1) / kPage : 0;
        pages_pre[b] = n;
        mine.x += n;
        mine.y += n > 0;
    }
    int2 tot;
    const int2 incl = block_inclusive_scan2(mine, wave_tot, &tot);
    int pages_off = incl.x - mine.x, ne_off = incl.y - mine.y;
    for (int b = b_lo; b < b_hi; ++b) {
        const int n = pages_pre[b];
        pages_pre[b] = pages_off;
        nonempty_pre[b] = ne_off;
        pages_off += n;
        ne_off += n > 0;
    }
    if (t == 0) {
        pages_pre[batch] = tot.x;
        nonempty_pre[batch] = tot.y;
    }
    __syncthreads();

    PlanView v;
    v.pages_pre = pages_pre;
    v.nonempty_pre = nonempty_pre;
    v.batch = batch;
    v.c = c;
    v.total = (int64_t)tot.x + (int64_t)c * tot.y;
    v.parts_eff = v.total < num_parts ? v.total : num_parts;

    for (int p = t; p < num_parts; p += kPlanThreads) {
        int32_t row[kMetaInts];
        v.part_row(p, row);
        for (int k = 0; k < kMetaInts; ++k) meta[p * kMetaInts + k] = row[k];
    }

    int2 my_splits = {0, 0};
    for (int b = b_lo; b < b_hi; ++b) my_splits.x += v.splits_of(b);
    int2 tot_splits;
    int off = block_inclusive_scan2(my_splits, wave_tot, &tot_splits).x - my_splits.x;
    for (int b = b_lo; b < b_hi; ++b) {
        split_base[b] = off;
        off += v.splits_of(b);
    }
    if (t == 0) split_base[batch] = tot_splits.x;
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
