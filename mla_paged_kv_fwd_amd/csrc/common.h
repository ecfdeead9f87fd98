// Shared definitions for the libmla HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kDQk = 576;             // latent 512 + decoupled RoPE 64
constexpr int kDV = 512;              // value = first 512 dims of the key row
constexpr int kPage = 64;             // tokens per cache page
constexpr int kTokBytesBf16 = 2 * kDQk;  // 1152
constexpr int kTokBytesFp8 = 656;     // 512 e4m3 + 4 fp32 scales + 64 bf16
constexpr int kFp8ScalesAt = 512;
constexpr int kFp8RopeAt = 528;
constexpr int kMetaInts = 8;
constexpr int kMaxBatch = 16384;
constexpr int kMaxParts = 16384;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Everything the attention kernels read.  Device pointers.
struct DecodeArgs {
    const uint16_t *q;          // bf16 [batch][M][576], M = s_q * h_q
    const unsigned char *kv;    // bf16 [pages][64][576] or fp8 [pages][64][656]
    const int32_t *block_table; // [batch][bt_stride]
    const int32_t *seqlens;     // [batch]
    const int32_t *meta;        // [num_parts][8]
    const int32_t *split_base;  // [batch + 1]
    float *o_part;              // fp32 [slots][M][512]
    float *lse_part;            // fp32 [slots][M]
    uint16_t *out;              // bf16 [batch][M][512]
    float *lse;                 // fp32 [batch][M]
    int64_t bt_stride;
    int batch, s_q, h_q, M;
    int num_parts;
    int row_groups;             // M / rows per work-group
    float scale_log2;           // softmax_scale * log2(e)
    int causal;
    int token_list;             // 64-row kernels: block_table holds token-id lists
};

// Split-KV plan: work of one part, computed identically on host and device
// from the request prefix sums.  E(b) = pages_pre[b+1] + c * nonempty_pre[b+1]
// is the cost-line position where request b ends.
struct PlanView {
    const int32_t *pages_pre;    // [batch + 1] exclusive prefix of ceil(L/64)
    const int32_t *nonempty_pre; // [batch + 1] exclusive prefix of (L > 0)
    int batch;
    int c;                       // overhead units per request segment
    int64_t total;               // T
    int64_t parts_eff;           // min(num_parts, T)

    __host__ __device__ int64_t end_of(int b) const {
        return (int64_t)pages_pre[b + 1] + (int64_t)c * nonempty_pre[b + 1];
    }
    __host__ __device__ int npages(int b) const { return pages_pre[b + 1] - pages_pre[b]; }
    __host__ __device__ int64_t start_of_pages(int b) const {  // position of page 0
        return (int64_t)pages_pre[b] + (int64_t)c * nonempty_pre[b] + c;
    }
    // first b with end_of(b) > x  (end_of is non-decreasing); batch if none
    __host__ __device__ int first_end_above(int64_t x) const {
        int lo = 0, hi = batch;
        while (lo < hi) {
            int mid = (lo + hi) >> 1;
            if (end_of(mid) > x) hi = mid; else lo = mid + 1;
        }
        return lo;
    }
    // first b with end_of(b) >= x
    __host__ __device__ int first_end_at_least(int64_t x) const {
        int lo = 0, hi = batch;
        while (lo < hi) {
            int mid = (lo + hi) >> 1;
            if (end_of(mid) >= x) hi = mid; else lo = mid + 1;
        }
        return lo;
    }
    __host__ __device__ int64_t part_of(int64_t pos) const { return pos * parts_eff / total; }

    // meta row of part p (8 ints)
    __host__ __device__ void part_row(int p, int32_t *row) const {
        for (int k = 0; k < kMetaInts; ++k) row[k] = 0;
        row[0] = -1;
        if (total == 0 || p >= parts_eff) return;
        int64_t lo = ((int64_t)p * total + parts_eff - 1) / parts_eff;
        int64_t hi = ((int64_t)(p + 1) * total + parts_eff - 1) / parts_eff;
        int b1 = first_end_above(lo);
        if (b1 >= batch) return;
        int64_t s1 = start_of_pages(b1);
        int64_t pos1 = lo > s1 ? lo : s1;
        if (pos1 >= hi) return;  // only overhead units in this part
        int b2 = first_end_at_least(hi);
        int j2;
        if (b2 < batch && npages(b2) > 0 && hi - 1 >= start_of_pages(b2)) {
            j2 = (int)(hi - 1 - start_of_pages(b2));
        } else {
            // hi - 1 falls in b2's overhead: last page is that of the previous
            // request with pages
            int64_t prev_end = (b2 < batch) ? (end_of(b2) - (npages(b2) > 0 ? c + npages(b2) : 0))
                                            : end_of(batch - 1);
            b2 = first_end_at_least(prev_end);
            j2 = npages(b2) - 1;
        }
        row[0] = b1;
        row[1] = (int)(pos1 - s1);
        row[2] = b2;
        row[3] = j2;
        row[4] = (int)(p - part_of(s1));
    }
    // number of parts touching request b
    __host__ __device__ int splits_of(int b) const {
        int n = npages(b);
        if (n == 0 || total == 0) return 0;
        int64_t s = start_of_pages(b);
        return (int)(part_of(s + n - 1) - part_of(s)) + 1;
    }
};

__host__ __device__ inline int plan_overhead(int s_q, int h_q) { return 1 + (s_q * h_q) / 64; }

}  // namespace mla
